// FP8 (OCP e4m3) forward attention for gfx950: block quantiser and fp8 attention kernel.
//
// Method (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention", Deep Dive "FP8
// accuracy controls" and "FP8 layout conformance"): one fp32 scale per Q, K or V block;
// Q and K are multiplied by the same orthogonal M = diag(s) H_d / sqrt(d) (random signs and
// a Hadamard matrix, O(d log d)) so that scores are unchanged while outliers spread over
// the head dimension; the second product's operand layout is made to match the first
// product's accumulator by permuting V's rows inside the kernel. The enterprise post ("FP8
// Accumulation") fixes 64-row blocks and fp32 scales.
//
// fp8_quant_kernel: one workgroup per (batch, head, 64-row block); 4 threads per row with
//   d/4 contiguous elements each. Signs, then the Hadamard butterfly (log2(d/4) in-thread
//   stages and 2 stages across the row's 4 lanes), times 1/sqrt(d); block amax by wave and
//   LDS reduction; descale = amax/448 (1 for an all-zero block); code = RNE(y / descale)
//   after clamping to +-448 (the hardware convert is not saturating). Per-tensor mode (the
//   single-scale baseline that block quantisation is compared with): the same kernel
//   writes each block's amax, one workgroup reduces them to the tensor's descale and
//   writes it to every block's slot, and the kernel runs again to encode with it.
//
// fwd_fp8_kernel: the bf16 forward's structure with v_mfma_f32_32x32x64_f8f6f4 (e4m3 x
//   e4m3, fp32 accumulate) on 64-key tiles (one K and one V scale block each): DMA ring,
//   S^T = K8 Q8^T with one query per lane, P~ packed to fp8 straight from the score
//   accumulators, V^T gathered by 8-bit transpose reads in the accumulators' key order,
//   the V descale folded into the exp2 argument (details at the kernel).
#include "attn_launch.h"
#include "attn_lds.h"

namespace attn {

namespace {

constexpr float kE4m3Max = 448.0f;

template <bool BF16>
__device__ __forceinline__ void unpack2q(uint32_t x, float& lo, float& hi) {
  if constexpr (BF16) {
    lo = __uint_as_float(x << 16);
    hi = __uint_as_float(x & 0xffff0000u);
  } else {
    lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
    hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
}

__device__ __forceinline__ uint32_t cvt4_fp8(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -kE4m3Max), kE4m3Max); }

// ---------------------------------------------------------------- quantiser
// MODE kQuantBlock: the block's own descale, codes and descale written. kQuantAmax: only
// the block's amax (of the rotated values) is written, to the descale slot. kQuantFixed:
// codes with the descale already in the slot (which is left as it is).
constexpr int kQuantBlock = 0, kQuantAmax = 1, kQuantFixed = 2;
// Rotary position embedding of one row's EPT consecutive dims (pairs (2i, 2i+1) with
// i = first/2 .. ): pair i at position pos turns by pos * theta_i, theta_i = base^(-2i/d).
// The angle is formed and reduced modulo 2 pi in fp64, so it stays exact to about 1e-12 at
// any position below 2^31; only its sine and cosine and the 2x2 rotation are fp32.
template <int D, int EPT>
__device__ __forceinline__ void rope_row(float (&y)[EPT], int pos, int first, double log2_base) {
  constexpr double kTwoPi = 6.283185307179586232;    // fp64(2 pi)
  constexpr double kInvTwoPi = 0.15915494309189534561;
  double theta = exp2(-(double)first / D * log2_base);
  const double ratio = exp2(-2.0 / D * log2_base);
#pragma unroll
  for (int e = 0; e < EPT; e += 2) {
    const double ang = (double)pos * theta;
    const double r = fma(-rint(ang * kInvTwoPi), kTwoPi, ang);
    float sn, cs;
    sincosf((float)r, &sn, &cs);
    const float a = y[e], b = y[e + 1];
    y[e] = a * cs - b * sn;
    y[e + 1] = a * sn + b * cs;
    theta *= ratio;
  }
}

template <bool BF16, int D, int MODE, bool ROPE>
__global__ __launch_bounds__(256) void fp8_quant_kernel(Fp8QuantParams p) {
  constexpr int EPT = D / 4;   // elements per thread (4 threads per row)
  const int tid = threadIdx.x, t = tid & 3, rloc = tid >> 2;
  const int H = p.H, N = p.N;
  const int nblk = (N + 63) / 64;
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int h = bh % H, b = bh / H;
  const int row = blk * 64 + rloc;

  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const size_t head_off = ((size_t)b * N * H + h) * D;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D * 2;
  const auto rx = make_rsrc((const char*)p.x + head_off * 2, nrec);
  const auto r8 = make_rsrc(p.x8 + head_off, (uint32_t)N * H * D - (uint32_t)h * D);

  float y[EPT];
#pragma unroll
  for (int c = 0; c < EPT / 8; ++c) {
    const u32x4 v = buf_load16(rx, (uint32_t)row * row_bytes + (t * EPT + 8 * c) * 2);
#pragma unroll
    for (int w = 0; w < 4; ++w) unpack2q<BF16>(v[w], y[8 * c + 2 * w], y[8 * c + 2 * w + 1]);
  }
  if constexpr (ROPE) rope_row<D, EPT>(y, row, t * EPT, p.rope_log2_base);
  if (p.rotate) {
    // this thread's sign bits: dims t*EPT .. +EPT-1, bit e of word e/32 (EPT/32 words, or the
    // right half of one word when EPT = 16)
    constexpr int NW = (EPT + 31) / 32;
    uint32_t sw[NW];
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int b0 = t * EPT + 32 * k;
      sw[k] = p.neg[b0 >> 5] >> (b0 & 31);
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      y[e] = __uint_as_float(__float_as_uint(y[e]) ^ ((sw[e >> 5] << (31 - (e & 31))) & 0x80000000u));
    // Sylvester Hadamard in natural order: pair (i, i + len) -> (x_i + x_j, x_i - x_j).
#pragma unroll
    for (int len = 1; len < EPT; len <<= 1)
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if ((i & len) == 0) {
          const float a = y[i], c = y[i + len];
          y[i] = a + c;
          y[i + len] = a - c;
        }
    // the last two stages pair the row's 4 lanes (a quad): lane t^1, then lane t^2, read
    // with DPP quad permutations; the lane with bit m set keeps the difference
    {
      const float sg = (t & 1) ? -1.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        y[e] = fmaf(sg, y[e], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y[e]), 0xB1, 0xF, 0xF, false)));
    }
    {
      const float sg = (t & 2) ? -1.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        y[e] = fmaf(sg, y[e], __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y[e]), 0x4E, 0xF, 0xF, false)));
    }
    const float inv_sqrt_d = (D == 64) ? 0.125f : (D == 256) ? 0.0625f : 0.088388347648318440550f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) y[e] *= inv_sqrt_d;
  }
  float* const ds_slot = p.descale + ((size_t)b * H + h) * nblk + blk;
  float descale;
  if constexpr (MODE == kQuantFixed) {
    descale = *ds_slot;
  } else {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) amax = fmaxf(amax, fabsf(y[e]));
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
    __shared__ float red[4];
    if ((tid & 63) == 0) red[tid >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if constexpr (MODE == kQuantAmax) {
      if (tid == 0) *ds_slot = amax;
      return;
    }
    descale = amax > 0.f ? amax / kE4m3Max : 1.0f;
  }

  // y / descale, correctly rounded to fp32: the product with the fp64 reciprocal carries a
  // relative error below 2^-52, while a quotient of two fp32 numbers lies at least about
  // 2^-49 (relative) from any fp32 rounding boundary, so rounding that product to fp32 gives
  // the IEEE quotient.
  const double rds = 1.0 / (double)descale;
  auto quot = [&](float v) { return (float)((double)v * rds); };
  uint32_t codes[EPT / 4];
#pragma unroll
  for (int w = 0; w < EPT / 4; ++w)
    codes[w] = cvt4_fp8(clamp448(quot(y[4 * w])), clamp448(quot(y[4 * w + 1])),
                        clamp448(quot(y[4 * w + 2])), clamp448(quot(y[4 * w + 3])));
#pragma unroll
  for (int c = 0; c < EPT / 16; ++c)
    buf_store16(r8, (uint32_t)row * H * D + t * EPT + 16 * c,
                u32x4{codes[4 * c], codes[4 * c + 1], codes[4 * c + 2], codes[4 * c + 3]});
  if (MODE == kQuantBlock && tid == 0) *ds_slot = descale;
}

// One workgroup: the tensor's descale from the n block amaxes in d (written by kQuantAmax),
// written back to all n slots: fp32(amax / 448), or 1 if the whole tensor is zero. Every
// thread has read its slots before the barrier that precedes the first write.
__global__ __launch_bounds__(1024) void fp8_tensor_scale_kernel(float* d, int n) {
  const int tid = threadIdx.x;
  float amax = 0.f;
  for (int i = tid; i < n; i += 1024) amax = fmaxf(amax, d[i]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  __shared__ float red[16];
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) amax = fmaxf(amax, red[w]);
  const float descale = amax > 0.f ? amax / kE4m3Max : 1.0f;
  for (int i = tid; i < n; i += 1024) d[i] = descale;
}

// ---------------------------------------------------------------- fp8 attention
template <int D> struct Fp8Cfg;
// WAVES: waves per workgroup (one workgroup per CU); STAGES: depth of the K and V rings.
template <> struct Fp8Cfg<64> { static constexpr int WAVES = 8, STAGES = 3; };
template <> struct Fp8Cfg<128> { static constexpr int WAVES = 8, STAGES = 3; };
template <> struct Fp8Cfg<256> { static constexpr int WAVES = 4, STAGES = 3; };
constexpr int kQW8 = 32;              // query rows per wave
template <int D> constexpr int fp8_rows() { return Fp8Cfg<D>::WAVES * kQW8; }
constexpr int kBC8 = 64;              // keys per tile: one K and one V scale block
constexpr float kTau8 = 2.5f;         // lazy-rescale threshold (log2 units): 64 * 2^2.5 = 362 < 448
constexpr float kPScale = 64.0f;      // P~ * 64 * dv/dv_max is the fp8 PV operand
constexpr float kLn2 = 0.69314718055994530942f;
// K tiles: row-major e4m3 rows of D bytes at pitch D + 16 (the K row reads of a 16-lane
// group fall on disjoint banks). V tiles: pitch D + 32 with rows exchanged by swap23 (see
// vt8_lane_off), which makes the transpose reads conflict-free.
template <int D> __host__ __device__ constexpr int f8_pitch() { return D + 16; }
template <int D> __host__ __device__ constexpr int f8_vpitch() { return D + 32; }

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// The same with B multiplied by 2^(code_b - 127) (E8M0 scale code; A unscaled, code 127).
__device__ __forceinline__ f32x16 mfma_f8_scaled(const i32x8& a, const i32x8& b, f32x16 c, int code_b) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, code_b);
}

// Row sums of the e4m3 P operand on the matrix core. The 32x32x64 P^T operand (lane l: query
// l%32, keys of half l/32) read as the B operand of a 16x16x128 product has lane l in column
// l%16 and K-chunk l/16, i.e. chunk c holds query 16*(c%2) + l%16. An A operand of ones on
// the chunks of one parity per row picks one query per output row; choosing, for the rows
// 4*(l/16) .. +3 that lane l receives, the parity of lane l's own query gives every lane the
// sum of its query's 64 rounded operands (in all four result registers).
__device__ __forceinline__ i32x8 rowsum_selector(int lane) {
  const int m = lane & 15, c = lane >> 4;
  const int one4 = 0x38383838;   // four e4m3 ones
  const int v = ((c & 1) == ((m >> 2) & 1)) ? one4 : 0;
  return i32x8{v, v, v, v, v, v, v, v};
}
__device__ __forceinline__ float rowsum_f8(const i32x8& sel, const i32x8& p) {
  const f32x4 r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, p, f32x4{}, 0, 0, 0, 0, 0, 0);
  return r[0];
}

// K operand of S^T = K Q^T: lane l holds key row kb*32 + l%32, dims 64*ks + 32*(l/32) .. +31.
template <int P>
__device__ __forceinline__ int k8_lane_off(int lane) { return (lane & 31) * P + (lane >> 5) * 32; }
template <int P>
__device__ __forceinline__ i32x8 lds_k8(const char* lane_base, int kb, int ks) {
  const char* a = lane_base + kb * 32 * P + ks * 64;
  const u32x4 x = *(const u32x4*)a, y = *(const u32x4*)(a + 16);
  return i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}
// V^T operand of O^T += V^T P^T, gathered from the row-major V tile by four 8-bit transpose
// reads (ds_read_b64_tr_b8: within each 16-lane group, lane i receives byte i%8 of the 8-byte
// pieces of source lanes 2e + i/8, e = 0..7, as its byte e). The P operand taken straight
// from two 32-key score accumulators holds, in byte b of lane half h, key
// 32*(b/16) + 8*((b%16)/4) + 4*h + b%4; so source lane s of read j points at key
// 16j + 8*(s/8) + 4*h + (s/2)%4 and dims 16*((l/16)%2) + 8*(s%2), and lane l receives dim
// l%32 (plus 32*i for output block i) of exactly the keys of its P bytes 8j .. 8j+7.
// The tile's rows are stored exchanged by swap23, so key 16j + 8a + 4h + c sits at LDS row
// 16j + 8h + 4a + c: the 32 lanes of one half (one LDS pass of 8-byte reads) gather 8
// consecutive rows, 32 bytes each, and at a pitch of D + 32 bytes (an odd multiple of 32
// modulo 256) those 8 pieces cover all 64 banks once.
template <int P>
__device__ __forceinline__ int vt8_lane_off(int lane) {
  const int s = lane & 15, h = lane >> 5;
  return (8 * h + 4 * (s >> 3) + ((s >> 1) & 3)) * P + 16 * ((lane >> 4) & 1) + 8 * (s & 1);
}
template <int P>
__device__ __forceinline__ i32x8 lds_vt8(const char* lane_base, int i) {
  i32x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) i32x2*)(lane_base + 16 * j * P + 32 * i));
    r[2 * j] = t[0];
    r[2 * j + 1] = t[1];
  }
  return r;
}

// One workgroup per (query tile, head, batch), the bf16 forward's structure in fp8:
//  * S^T = K8 Q8^T (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulate): lane owns a query; the Q
//    and K descales fold into one per-lane, per-tile coefficient of the exp2 argument
//    (scores scaled by scale*log2(e)*dq*dk).
//  * One 64-key PV product consumes exactly the tile's two 32-key score accumulators (32 fp8
//    bytes per lane) against the V^T operand read by transpose reads (see lds_vt8).
//  * The V descale of the tile enters the exp2 argument as log2(64*dv/dv_max), dv_max being
//    the head's largest V descale; the row sum l counts the unweighted P~, and the epilogue
//    multiplies O by dv_max/64/l. The lazy-rescale threshold is 2^2.5, so the fp8 operand
//    P~*64*dv/dv_max stays in [0, 362], inside e4m3's range (448).
//  * K and V tiles arrive by DMA in a three-stage LDS ring; the pipelined loop forms
//    S(j+1) on the matrix cores while the VALU exponentiates tile j, then P~(j) V(j) while
//    the VALU sums tile j and takes the row maximum of tile j+1.
template <bool OUT_BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * Fp8Cfg<D>::WAVES, 1) void fwd_fp8_kernel(Fp8FwdParams p) {
  constexpr int kWaves = Fp8Cfg<D>::WAVES;
  constexpr int NS = Fp8Cfg<D>::STAGES;
  constexpr int kBR = fp8_rows<D>();
  constexpr int BC = kBC8;
  constexpr int NKB = BC / 32;       // 32-key score blocks per tile
  constexpr int NKS = D / 64;        // k-steps of the score product
  constexpr int NDB = D / 32;        // 32-dim output blocks
  constexpr int P8 = f8_pitch<D>(), PV8 = f8_vpitch<D>();
  using Plan = DmaPlanBytes<D, BC, P8, kWaves>;
  using VPlan = DmaPlanBytes<D, BC, PV8, kWaves>;
  constexpr int TB = Plan::BYTES, TBV = VPlan::BYTES;
  constexpr int KMIN = Plan::NI / kWaves;   // may be 0 (small tiles): such waves issue no DMA
  constexpr int KMINV = VPlan::NI / kWaves;
  // Ping-pong (two waves per SIMD): the second wave of each SIMD runs the P~V half of every
  // fast tile one barrier interval late, so that on each SIMD one wave exponentiates while
  // the other multiplies; V(j) is then read one interval later, which one more V stage covers.
  constexpr bool PP = kWaves == 8;
  constexpr int VS = NS + (PP ? 1 : 0);
  // One LDS array: the ring stages, then a slot for the per-wave maxima of the V descales.
  // (With a second __shared__ variable the compiler gives every access to this one the same
  // alias scope, loses the restrict scopes below, and waits for all DMA before LDS reads.)
  // Then the tile descriptor table (below) in the rest of the CU's 160 KiB.
  constexpr int DT_OFF = NS * TB + VS * TBV + 4 * kWaves;
  constexpr int DT_MAX = (160 * 1024 - DT_OFF) / 16;
  static_assert(DT_OFF % 16 == 0 && DT_MAX > 0, "descriptor table placement");
  __shared__ __attribute__((aligned(1024))) char smem[DT_OFF + 16 * DT_MAX];
  float* const red = (float*)(smem + NS * TB + VS * TBV);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H, N = p.N;
  const int nqt = (N + kBR - 1) / kBR;
  const int nblk = (N + 63) / 64;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const int qt = CAUSAL ? nqt - 1 - qi : qi;
  const int q0 = qt * kBR + wave * kQW8;
  const int qrow = q0 + l32;

  const uint32_t row_bytes = (uint32_t)H * D;
  const size_t head_off = ((size_t)b * N * H + h) * D;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D;
  const auto rq = make_rsrc(p.q8 + head_off, nrec);
  const uint32_t orow = (uint32_t)H * D * 2;
  const auto ro = make_rsrc((char*)p.o + head_off * 2, (uint32_t)N * orow - (uint32_t)h * D * 2);
  const float* dq_h = p.dq + ((size_t)b * H + h) * nblk;
  const float* dk_h = p.dk + ((size_t)b * H + h) * nblk;
  const float* dv_h = p.dv + ((size_t)b * H + h) * nblk;
  // Per-tile K and V descales by scalar loads: a uniform address in the constant address
  // space (the kernel never writes them). A vector load would count on vmcnt with the tile
  // DMA, and the wait for its value would also wait for every DMA issued before the use.
  using cfloat = const __attribute__((address_space(4))) float;
  cfloat* dk_s = (cfloat*)dk_h;
  cfloat* dv_s = (cfloat*)dv_h;

  // largest V descale of the head (before any DMA is in flight)
  float dvm = 0.f;
  for (int i = tid; i < nblk; i += 64 * kWaves) dvm = fmaxf(dvm, dv_h[i]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) dvm = fmaxf(dvm, __shfl_xor(dvm, m));
  if (lane == 0) red[wave] = dvm;
  __syncthreads();
  dvm = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) dvm = fmaxf(dvm, red[w]);
  // A head whose V descales are all zero has V = 0: any positive reference gives O = 0.
  if (!(dvm > 0.f)) dvm = 1.0f;

  // Q^T operand: lane holds query q0 + l32, dims 64*ks + 32*hf .. +31.
  i32x8 qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const u32x4 a = buf_load16(rq, (uint32_t)qrow * row_bytes + 64 * ks + 32 * hf);
    const u32x4 c = buf_load16(rq, (uint32_t)qrow * row_bytes + 64 * ks + 32 * hf + 16);
    qreg[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  }
  const float cq = p.c * (qrow < N ? dq_h[qrow >> 6] : 1.0f);

  const int kend = CAUSAL ? min(N, (qt + 1) * kBR) : N;
  const int nkt = (kend + BC - 1) / BC;
  const int nkt_w = q0 >= N ? 0 : CAUSAL ? min(nkt, (q0 + kQW8 - 1) / BC + 1) : nkt;
  auto is_edge = [&](int j) { const int k0 = j * BC; return (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0); };
  // Stage offsets pass through readfirstlane: opaque to loop strength reduction.
  auto kst = [&](int j) { return smem + __builtin_amdgcn_readfirstlane((j % NS) * TB); };
  auto vst = [&](int j) { return smem + NS * TB + __builtin_amdgcn_readfirstlane((j % VS) * TBV); };
  uint32_t voff[Plan::NPW], vvoff[VPlan::NPW];
  dma_init<Plan, kWaves>(voff, row_bytes, wave, lane);
  dma_init<VPlan, kWaves, 0, true>(vvoff, row_bytes, wave, lane);
  const char* kbase = (const char*)p.k8 + head_off;
  const char* vbase = (const char*)p.v8 + head_off;
  auto dma_k = [&](int t) { dma_issue<Plan, kWaves>(voff, kst(t), kbase, t * BC, row_bytes, nrec, wave); };
  auto dma_v = [&](int t) { dma_issue<VPlan, kWaves>(vvoff, vst(t), vbase, t * BC, row_bytes, nrec, wave); };

  // DMA schedule as in the bf16 forward: the prologue requests K(0), then V(t), K(t+1) for
  // t = 0 .. NS-2; iteration j requests V(j+NS-1), K(j+NS); before iteration j, K(j+1) and
  // V(j) must have landed.
  // this wave's DMA instructions per K tile and per V tile
  const int n_w = KMIN + (wave < Plan::NI % kWaves ? 1 : 0);
  const int n_wv = KMINV + (wave < VPlan::NI % kWaves ? 1 : 0);
  constexpr int KEEP_MAX = (NS - 2) * (KMIN + KMINV + 2);
  auto wait_before = [&](int j) {
    int keep = 0;
#pragma unroll
    for (int t = 1; t <= NS - 2; ++t) keep += (j + t < nkt ? n_wv : 0) + (j + t + 1 < nkt ? n_w : 0);
    // Away from the end of the key range every tile of the batch exists: keep the count
    // of the waves with the fewest DMA instructions, a constant. The other waves then also
    // wait for the first one or two of their batch, issued at the start of the tile
    // (waiting longer is always safe); a count chosen at run time would cost a chain of
    // compares and branches per tile.
    if (j + NS - 1 < nkt) wait_dma_keep<(NS - 2) * (KMIN + KMINV)>();
    else wait_dma_keep_rt<KEEP_MAX>(keep);
  };
  // per-tile descale factors, loaded one tile ahead (t < nkt <= nblk)
  auto load_desc = [&](int t, float& dk, float& dv) {
    dk = dk_s[t];
    dv = dv_s[t];
  };
  float dk_c, dv_c;   // descales of tile 0 (later tiles: tile_desc below)
  load_desc(0, dk_c, dv_c);
  // The weight 64 * dv/dv_max of a tile's P~ is split as 2^e * w, w in [32, 64): w enters the
  // exp2 argument as its log2 (so every tile's e4m3 operand P~ w spans the same range, whatever
  // its V scale), and 2^e is the E8M0 scale code 127 + e that the PV product applies to that
  // operand exactly. The row sums take P~ and the rounded operands through 1/w. A V block
  // with descale 0 (all zeros) gets w = 64 and code 0 (2^-127): its keys still count in both
  // row sums, and its zero codes add nothing to O. Formed one tile ahead, off the path from
  // the tile barrier to the first exponential.
  const float inv_dvm = 1.0f / dvm;
  float logw_c, rw_c;
  int sc_c;
  auto weight_of = [&](float dv, float& logw, float& rw, int& code) {
    const float r = dv * inv_dvm;   // in [0, 1]
    const bool normal = r >= 0x1p-126f;
    const float w = normal ? kPScale * __builtin_amdgcn_frexp_mantf(r) : kPScale;
    code = normal ? 127 + __builtin_amdgcn_frexp_expf(r) : 0;
    logw = fast_log2(w);
    rw = __builtin_amdgcn_rcpf(w);
  };
  auto set_weight = [&](float dv) { weight_of(dv, logw_c, rw_c, sc_c); };
  // Tile descriptors: the K descale and the V weight split (log2 w, 1/w, code) of every key
  // tile, formed once per workgroup into the LDS after the ring when the head's tiles fit
  // (then a tile costs one broadcast 16-byte read instead of two scalar loads, a frexp pair, a
  // log2 and a reciprocal), else formed per tile as the iterations need them.
  f32x4* const dtab = (f32x4*)(smem + DT_OFF);
  const bool use_dtab = nkt <= DT_MAX;
  auto tile_desc = [&](int t, float& dk, float& logw, float& rw, int& code) {
    if (use_dtab) {
      const f32x4 v = dtab[t];
      dk = v[0];
      logw = v[1];
      rw = v[2];
      code = __float_as_int(v[3]);
    } else {
      float dv;
      load_desc(t, dk, dv);
      weight_of(dv, logw, rw, code);
    }
  };

  dma_k(0);
#pragma unroll
  for (int t = 0; t <= NS - 2; ++t) {
    if (t < nkt) dma_v(t);
    if (t + 1 < nkt) dma_k(t + 1);
  }
  // the descriptor table, published by the barrier before the first tile (its loads are
  // issued after the first tiles' DMA, so waiting for them holds nothing else up)
  if (use_dtab) {
    for (int t = tid; t < nkt; t += 64 * kWaves) {
      float lw, rwt;
      int code;
      weight_of(dv_h[t], lw, rwt, code);
      dtab[t] = f32x4{dk_h[t], lw, rwt, __int_as_float(code)};
    }
  }
  // Q (and its descale) waited for here, not inside the tile loop, and only now: the load
  // and the first tiles' DMA share one HBM round trip
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) settle(qreg[ks]);
  settle(cq);

  set_weight(dv_c);
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  // l_run: the row sum of the unrounded P~ (lane partial over its half of each tile), which
  // gives L; l_rnd: the row sum of the e4m3-rounded operands divided by their weights, which
  // normalises O, so that O's weights are exactly the operands the PV product used.
  float m_run = -INFINITY, l_run = 0.f, l_rnd = 0.f;
  const i32x8 sel = rowsum_selector(lane);
  const int k_lane = k8_lane_off<P8>(lane), v_lane = vt8_lane_off<PV8>(lane);

  wait_before(0);
  __syncthreads();

  auto tile_scores = [&](f32x16 (&sc)[NKB], const char* kl) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) sc[kb] = mfma_f8(lds_k8<P8>(kl, kb, ks), qreg[ks], sc[kb]);
    }
  };
  auto tile_mask = [&](f32x16 (&sc)[NKB], int k0) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= N || (CAUSAL && key > qrow)) sc[kb][r] = -INFINITY;
      }
  };
  auto tile_max = [&](const f32x16 (&sc)[NKB], float coef) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
    mx = xhalf_max(mx);
    return mx == -INFINITY ? -INFINITY : mx * coef;
  };

  // prologue: scores and maximum of tile 0
  f32x16 sc[NKB], sn[NKB];
  float mx_next = -INFINITY;
  float coef_c = cq * dk_c;   // coefficient of the tile held in sc
  if (nkt_w > 0) {
    tile_scores(sc, kst(0) + k_lane);
    if (is_edge(0)) tile_mask(sc, 0);
    mx_next = tile_max(sc, coef_c);
  }
  // the first prefetch overwrites the stage of K(0), which the prologue just read
  ring_barrier();

  auto prefetch = [&](int j) {
    if (j + NS - 1 < nkt) dma_v(j + NS - 1);
    if (j + NS < nkt) dma_k(j + NS);
  };
  auto end_tile = [&](int j) {
    wait_before(j + 1);
    ring_barrier();
  };
  auto rescale = [&]() {
    const float m_cand = fmaxf(m_run, mx_next);
    if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kTau8)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_cand);
      m_run = m_cand;
      l_run *= alpha;
      l_rnd *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
  };

  // Interior tiles, pipelined with the instruction order written out, in one of two forms.
  // Ping-pong (eight waves, d <= 128): block 1 issues one S(j+1) MFMA per step with EPS_P
  // exponentials of tile j under each, packed to fp8 four at a time and added to the row sum
  // (two partial sums) as they come, so that the fp32 P~ values do not stay live into block
  // 2; block 2 issues one P~(j)V(j) MFMA per step (one per 32-dim output block), the rounded
  // operands' row sum, and the row maximum of tile j+1. The two waves of a SIMD run the
  // blocks one barrier interval apart, so one's exponentials meet the other's P~V MFMAs.
  // One wave per SIMD (four waves, d = 256): the softmax work of a tile is split over two
  // iterations so that both blocks carry VALU work beside their MFMAs (a wave that issues
  // VALU work alone runs at about half the SIMD's VALU rate). Block 1 of tile j: one S(j+1)
  // MFMA per step and the exponentials of tile j's second key block. Block 2: one P~(j)V(j)
  // MFMA per step and the rounded operands' row sum; under its first MS steps the row
  // maximum of tile j+1 and the rescale decision for it, under the others the exponentials of
  // tile j+1's first key block into the other P~ operand buffer. The rescale of O and of the
  // row sums that the decision calls for is applied after the block, once P~(j)V(j) is in O.
  // (At d = 64 and 128 the split form measured 11% and 1% slower than the ping-pong, at
  // d = 256 14% faster than the unsplit form.)
  constexpr int S1 = NKB * NKS;
  constexpr int S2 = NDB;
  constexpr int PF = 2;
  constexpr int EPS_P = 16 * NKB / S1;                   // ping-pong form
  constexpr int MPS_P = 16 * NKB / S2;
  static_assert(EPS_P * S1 == 16 * NKB && MPS_P * S2 == 16 * NKB && EPS_P % 4 == 0 && MPS_P % 2 == 0, "step split");
  constexpr int EPS = 16 / S1;                           // split form: second-block exponentials per block-1 step
  constexpr int MS = S2 >= 2 ? S2 / 2 : 1;               // block-2 steps that fold the row maximum
  constexpr int MPS = 16 * NKB / MS;                     // scores folded into it per such step
  constexpr int EPS2 = 16 / (S2 - MS);                   // first-block exponentials per later step
  static_assert(NKB == 2 && EPS * S1 == 16 && MPS * MS == 16 * NKB && MPS % 2 == 0 && S2 > MS &&
                EPS2 * (S2 - MS) == 16 && EPS2 % 4 == 0, "step split");
  float dk_n, logw_n, rw_n;   // the next tile's descriptor
  int sc_n;
  // P~ operands. Kept across tiles: each conversion writes half of a word whose other half it
  // keeps, and the word it lands in belongs to a tile already consumed, so no register has to
  // be cleared first. The ping-pong form uses pka only; the split form alternates pka and pkb
  // (the next tile's first key block is made while the current one's operand is in use).
  i32x8 pka = {}, pkb = {};
  float psum_h = 0.f;                 // split form: row-sum part of the tile's first key block
  float bias_c = 0.f;                 // split form: exp2 bias of the tile, log2 w - m
  // kn, vc: K(jj+1) and V(jj) in LDS, this lane's bases; restrict, so that the compiler can
  // tell their reads from the stages the DMA in flight is filling (otherwise it waits for
  // every outstanding DMA before the first read, which drains the ring's prefetch each tile).
  auto fast_iter_pp = [&](auto late, int jj, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB], const char* __restrict__ kn,
                       const char* __restrict__ vc, char* __restrict__ kd, char* __restrict__ vd) __attribute__((always_inline)) {
    tile_desc(jj + 1 < nkt ? jj + 1 : jj, dk_n, logw_n, rw_n, sc_n);
    if (jj + NS - 1 < nkt) dma_issue<VPlan, kWaves>(vvoff, vd, vbase, (jj + NS - 1) * BC, row_bytes, nrec, wave);
    if (jj + NS < nkt) dma_issue<Plan, kWaves>(voff, kd, kbase, (jj + NS) * BC, row_bytes, nrec, wave);
    rescale();
    const float bias = logw_c - m_run;
    i32x8 kop[S1];
    float e[16 * NKB];
    float psum_a = 0.f, psum_b = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < PF && t < S1; ++t) kop[t] = lds_k8<P8>(kn, t % NKB, t / NKB);
#pragma unroll
    for (int t = 0; t < S1; ++t) {
      if (t + PF < S1) kop[t + PF] = lds_k8<P8>(kn, (t + PF) % NKB, (t + PF) / NKB);
      const int kb = t % NKB, ks = t / NKB;
      nxt[kb] = mfma_f8(kop[t], qreg[ks], ks == 0 ? f32x16{} : nxt[kb]);
#pragma unroll
      for (int u = 0; u < EPS_P; ++u) {
        const int i = EPS_P * t + u;
        e[i] = fast_exp2(fmaf(cur[i >> 4][i & 15], coef_c, bias));
        if ((i & 3) == 3) {
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e[i - 3], e[i - 2], pka[i >> 2], false);
          pka[i >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(e[i - 1], e[i], lo, true);
        }
        if (i & 1) psum_b += e[i]; else psum_a += e[i];
      }
      pin(psum_a);
      pin(psum_b);
      __builtin_amdgcn_sched_barrier(0);
    }
    // late waves: the barrier that ends this tile comes between the two blocks
    if constexpr (decltype(late)::value) end_tile(jj);
    const float coef_n = cq * dk_n;
    i32x8 vop[S2];
    float mx = -INFINITY;
    const float rsum = rowsum_f8(sel, pka);
#pragma unroll
    for (int t = 0; t < PF && t < S2; ++t) vop[t] = lds_vt8<PV8>(vc, t);
#pragma unroll
    for (int t = 0; t < S2; ++t) {
      if (t + PF < S2) vop[t + PF] = lds_vt8<PV8>(vc, t + PF);
      oacc[t] = mfma_f8_scaled(vop[t], pka, oacc[t], sc_c);
#pragma unroll
      for (int u = 0; u < MPS_P; u += 2) {
        const int i2 = MPS_P * t + u;
        mx = max3(mx, nxt[i2 >> 4][i2 & 15], nxt[(i2 + 1) >> 4][(i2 + 1) & 15]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = fmaf(psum_a + psum_b, rw_c, l_run);
    l_rnd = fmaf(rsum, rw_c, l_rnd);
    mx = xhalf_max(mx);
    mx_next = mx * coef_n;
    coef_c = coef_n;
    logw_c = logw_n;
    rw_c = rw_n;
    sc_c = sc_n;
    if constexpr (!decltype(late)::value) end_tile(jj);
  };
  // The split form's iteration (same operands).
  auto fast_iter = [&](auto late, int jj, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB], i32x8& pkc, i32x8& pkn,
                       const char* __restrict__ kn, const char* __restrict__ vc, char* __restrict__ kd,
                       char* __restrict__ vd) __attribute__((always_inline)) {
    tile_desc(jj + 1 < nkt ? jj + 1 : jj, dk_n, logw_n, rw_n, sc_n);
    if (jj + NS - 1 < nkt) dma_issue<VPlan, kWaves>(vvoff, vd, vbase, (jj + NS - 1) * BC, row_bytes, nrec, wave);
    if (jj + NS < nkt) dma_issue<Plan, kWaves>(voff, kd, kbase, (jj + NS) * BC, row_bytes, nrec, wave);
    const float coef_n = cq * dk_n;
    i32x8 kop[S1];
    float e[16];
    float psum_a = 0.f, psum_b = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < PF && t < S1; ++t) kop[t] = lds_k8<P8>(kn, t % NKB, t / NKB);
#pragma unroll
    for (int t = 0; t < S1; ++t) {
      if (t + PF < S1) kop[t + PF] = lds_k8<P8>(kn, (t + PF) % NKB, (t + PF) / NKB);
      const int kb = t % NKB, ks = t / NKB;
      nxt[kb] = mfma_f8(kop[t], qreg[ks], ks == 0 ? f32x16{} : nxt[kb]);
#pragma unroll
      for (int u = 0; u < EPS; ++u) {
        const int i = EPS * t + u;   // element i of the second key block
        e[i] = fast_exp2(fmaf(cur[1][i], coef_c, bias_c));
        if ((i & 3) == 3) {
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e[i - 3], e[i - 2], pkc[4 + (i >> 2)], false);
          pkc[4 + (i >> 2)] = __builtin_amdgcn_cvt_pk_fp8_f32(e[i - 1], e[i], lo, true);
        }
        if (i & 1) psum_b += e[i]; else psum_a += e[i];
      }
      pin(psum_a);
      pin(psum_b);
      __builtin_amdgcn_sched_barrier(0);
    }
    // late waves: the barrier that ends this tile comes between the two blocks
    if constexpr (decltype(late)::value) end_tile(jj);
    i32x8 vop[S2];
    float mx = -INFINITY, m_new = m_run, alpha = 1.f, bias_n = 0.f;
    bool need = false;
    float en[16];
    float qsum_a = 0.f, qsum_b = 0.f;
    const float rsum = rowsum_f8(sel, pkc);
#pragma unroll
    for (int t = 0; t < PF && t < S2; ++t) vop[t] = lds_vt8<PV8>(vc, t);
#pragma unroll
    for (int t = 0; t < S2; ++t) {
      if (t + PF < S2) vop[t + PF] = lds_vt8<PV8>(vc, t + PF);
      oacc[t] = mfma_f8_scaled(vop[t], pkc, oacc[t], sc_c);
      if (t < MS) {
#pragma unroll
        for (int u = 0; u < MPS; u += 2) {
          const int i2 = MPS * t + u;
          mx = max3(mx, nxt[i2 >> 4][i2 & 15], nxt[(i2 + 1) >> 4][(i2 + 1) & 15]);
        }
        if (t == MS - 1) {
          // the maximum of tile jj+1 may move the reference (O and the sums follow below)
          const float m_cand = fmaxf(m_run, xhalf_max(mx) * coef_n);
          need = __builtin_amdgcn_ballot_w64(m_cand > m_run + kTau8) != 0;
          if (need) {
            alpha = fast_exp2(m_run - m_cand);
            m_new = m_cand;
          }
          bias_n = logw_n - m_new;
        }
      } else {
#pragma unroll
        for (int u = 0; u < EPS2; ++u) {
          const int i = EPS2 * (t - MS) + u;   // element i of tile jj+1's first key block
          en[i] = fast_exp2(fmaf(nxt[0][i], coef_n, bias_n));
          if ((i & 3) == 3) {
            const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(en[i - 3], en[i - 2], pkn[i >> 2], false);
            pkn[i >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(en[i - 1], en[i], lo, true);
          }
          if (i & 1) qsum_b += en[i]; else qsum_a += en[i];
        }
        pin(qsum_a);
        pin(qsum_b);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run = fmaf(psum_h + (psum_a + psum_b), rw_c, l_run);
    l_rnd = fmaf(rsum, rw_c, l_rnd);
    if (need) {
      l_run *= alpha;
      l_rnd *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
    m_run = m_new;
    psum_h = qsum_a + qsum_b;
    coef_c = coef_n;
    bias_c = bias_n;
    logw_c = logw_n;
    rw_c = rw_n;
    sc_c = sc_n;
    if constexpr (!decltype(late)::value) end_tile(jj);
  };
  int j = 0;
  if constexpr (PP) {
    auto fast_loop = [&](auto late) __attribute__((always_inline)) {
      for (; j + 2 < nkt_w && !is_edge(j + 2); j += 2) {
        fast_iter_pp(late, j, sc, sn, kst(j + 1) + k_lane, vst(j) + v_lane, kst(j + NS), vst(j + NS - 1));
        fast_iter_pp(late, j + 1, sn, sc, kst(j + 2) + k_lane, vst(j + 1) + v_lane, kst(j + 1 + NS), vst(j + NS));
      }
      if (j + 1 < nkt_w && !is_edge(j + 1)) {
        fast_iter_pp(late, j, sc, sn, kst(j + 1) + k_lane, vst(j) + v_lane, kst(j + NS), vst(j + NS - 1));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sc[kb] = sn[kb];
        ++j;
      }
    };
    // Waves w and w + kWaves/2 share a SIMD (waves are placed on the SIMDs round-robin).
    if (wave >= kWaves / 2) fast_loop(std::true_type{});
    else fast_loop(std::false_type{});
  } else {
    // Whether tile 0 runs the fast form (tiles 0 and 1 need no mask): then its reference is set
    // and its first key block exponentiated here, as the iteration before would have done.
    const bool fast0 = 1 < nkt_w && !is_edge(1);
    if (fast0) {
      rescale();
      bias_c = logw_c - m_run;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) x4[u] = fast_exp2(fmaf(sc[0][4 * g + u], coef_c, bias_c));
        psum_h += (x4[0] + x4[1]) + (x4[2] + x4[3]);
        pka[g] = (int)cvt4_fp8(x4[0], x4[1], x4[2], x4[3]);
      }
    }
    auto fast_loop = [&](auto late) __attribute__((always_inline)) {
      for (; j + 2 < nkt_w && !is_edge(j + 2); j += 2) {
        fast_iter(late, j, sc, sn, pka, pkb, kst(j + 1) + k_lane, vst(j) + v_lane, kst(j + NS), vst(j + NS - 1));
        fast_iter(late, j + 1, sn, sc, pkb, pka, kst(j + 2) + k_lane, vst(j + 1) + v_lane, kst(j + 1 + NS), vst(j + NS));
      }
      if (j + 1 < nkt_w && !is_edge(j + 1)) {
        fast_iter(late, j, sc, sn, pka, pkb, kst(j + 1) + k_lane, vst(j) + v_lane, kst(j + NS), vst(j + NS - 1));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sc[kb] = sn[kb];
        pka = pkb;
        ++j;
      }
    };
    fast_loop(std::false_type{});
  }
  // Remaining tiles, in order: masked tiles and the tail of the key range (waves with
  // nothing left to compute only take part in the ring bookkeeping). After split-form fast
  // iterations, tile j has its reference set and its first key block in pka.
  bool half = !PP && j > 0;
  for (; j < nkt; ++j) {
    tile_desc(j + 1 < nkt ? j + 1 : j, dk_n, logw_n, rw_n, sc_n);
    prefetch(j);
    if (j < nkt_w) {
      if (!half) rescale();
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      const float bias = logw_c - m_use;
      const bool edge = is_edge(j);
      i32x8 pk = pka;
      float psum = half ? psum_h : 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          if (half && kb == 0) continue;
          float e4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x = sc[kb][4 * r4 + u];
            e4[u] = fast_exp2(fmaf(x, coef_c, bias));
            if (edge && x == -INFINITY) e4[u] = 0.f;
            psum += e4[u];
          }
          pk[4 * kb + r4] = (int)cvt4_fp8(e4[0], e4[1], e4[2], e4[3]);
        }
      l_run = fmaf(psum, rw_c, l_run);
      l_rnd = fmaf(rowsum_f8(sel, pk), rw_c, l_rnd);
      // V(j) through a restrict pointer, as in the fast iteration
      [&](const char* __restrict__ vc) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[i] = mfma_f8_scaled(lds_vt8<PV8>(vc, i), pk, oacc[i], sc_c);
      }(vst(j) + v_lane);
      if (j + 1 < nkt_w) {
        tile_scores(sc, kst(j + 1) + k_lane);
        if (is_edge(j + 1)) tile_mask(sc, (j + 1) * BC);
        mx_next = tile_max(sc, cq * dk_n);
      }
    }
    coef_c = cq * dk_n;
    logw_c = logw_n;
    rw_c = rw_n;
    sc_c = sc_n;
    half = false;
    end_tile(j);
  }

  // O leaves through the ring's LDS (not the descale slot after it), each wave in its own
  // area, in as many column parts as the ring needs for the 16-bit rows (two at d = 128):
  // the last end_tile() waited for every DMA and passed a barrier after every wave's last
  // operand read.
  constexpr int RING = NS * TB + VS * TBV;
  constexpr int OPARTS = kWaves * RowStage<2 * D>::BYTES <= RING ? 1 : kWaves * RowStage<D>::BYTES <= RING ? 2 : 4;
  using OStage = RowStage<2 * D / OPARTS>;
  static_assert(kQW8 == 32 && NDB % OPARTS == 0 && kWaves * OStage::BYTES <= RING, "O staging fits the ring");
  if (nkt_w > 0) {
    const float l_tot = xhalf_sum(l_run);
    const float fac = dvm / kPScale / l_rnd;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    char* ost = smem + wave * OStage::BYTES;
#pragma unroll
    for (int part = 0; part < OPARTS; ++part) {
#pragma unroll
      for (int i = part * (NDB / OPARTS); i < (part + 1) * (NDB / OPARTS); ++i)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d0 = i * 32 + 8 * rr + 4 * hf;
          const u32x2 v = {pack2<OUT_BF16>(oacc[i][4 * rr + 0] * fac, oacc[i][4 * rr + 1] * fac),
                           pack2<OUT_BF16>(oacc[i][4 * rr + 2] * fac, oacc[i][4 * rr + 3] * fac)};
          OStage::put(ost, l32, (d0 - part * (D / OPARTS)) * 2, v);
        }
      OStage::store(ost, ro, (uint32_t)q0, orow, part * (2 * D / OPARTS), lane);
    }
    if (hf == 0 && qrow < N) p.lse[((size_t)b * H + h) * N + qrow] = (m_use + fast_log2(l_tot)) * kLn2;
  }
}

template <bool BF16, int D, bool ROPE>
hipError_t launch_qr(const Fp8QuantParams& p, hipStream_t s) {
  const int nblk = (p.N + 63) / 64;
  const dim3 grid((unsigned)(p.B * p.H * nblk));
  if (!p.per_tensor) {
    hipLaunchKernelGGL((fp8_quant_kernel<BF16, D, kQuantBlock, ROPE>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fp8_quant_kernel<BF16, D, kQuantAmax, ROPE>), grid, dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fp8_tensor_scale_kernel, dim3(1), dim3(1024), 0, s, p.descale, p.B * p.H * nblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_quant_kernel<BF16, D, kQuantFixed, ROPE>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_q(const Fp8QuantParams& p, hipStream_t s) {
  return p.rope ? launch_qr<BF16, D, true>(p, s) : launch_qr<BF16, D, false>(p, s);
}

template <bool OUT_BF16, int D, bool CAUSAL>
hipError_t launch_f(const Fp8FwdParams& p, hipStream_t s) {
  const int nqt = (p.N + fp8_rows<D>() - 1) / fp8_rows<D>();
  hipLaunchKernelGGL((fwd_fp8_kernel<OUT_BF16, D, CAUSAL>), dim3((unsigned)(p.B * p.H * nqt)),
                     dim3(64 * Fp8Cfg<D>::WAVES), 0, s, p);
  return hipGetLastError();
}

template <bool OUT_BF16, int D>
hipError_t launch_fc(bool causal, const Fp8FwdParams& p, hipStream_t s) {
  return causal ? launch_f<OUT_BF16, D, true>(p, s) : launch_f<OUT_BF16, D, false>(p, s);
}

}  // namespace

hipError_t launch_fp8_quantize(bool bf16, int d, const Fp8QuantParams& p, hipStream_t s) {
  switch (d) {
    case 64: return bf16 ? launch_q<true, 64>(p, s) : launch_q<false, 64>(p, s);
    case 128: return bf16 ? launch_q<true, 128>(p, s) : launch_q<false, 128>(p, s);
    case 256: return bf16 ? launch_q<true, 256>(p, s) : launch_q<false, 256>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_fp8(bool out_bf16, int d, bool causal, const Fp8FwdParams& p, hipStream_t s) {
  switch (d) {
    case 64: return out_bf16 ? launch_fc<true, 64>(causal, p, s) : launch_fc<false, 64>(causal, p, s);
    case 128: return out_bf16 ? launch_fc<true, 128>(causal, p, s) : launch_fc<false, 128>(causal, p, s);
    case 256: return out_bf16 ? launch_fc<true, 256>(causal, p, s) : launch_fc<false, 256>(causal, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
