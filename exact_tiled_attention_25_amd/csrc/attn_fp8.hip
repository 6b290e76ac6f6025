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
//   after clamping to +-448 (the hardware convert is not saturating).
//
// fwd_fp8_kernel: the bf16 forward's structure with v_mfma_f32_32x32x64_f8f6f4 (e4m3 x
//   e4m3, fp32 accumulate), 128-key tiles = two 64-key products.
//  * S^T = K8 Q8^T: lane owns a query; Q and K descales fold into one per-lane, per-64-key
//    coefficient of the exp2 argument (scores scaled by scale*log2(e)*dq*dk).
//  * One 64-key PV product consumes exactly two 32-key score accumulators (32 fp8 bytes per
//    lane). Byte b of lane half h is key 32*(b/16) + 8*((b%16)/4) + 4*h + b%4, so V^T sits
//    in LDS with position bits [5:2] = rotr4(key bits [5:2]).
//  * The V descale of each 64-key block enters the exp2 argument as log2(64*dv/dv_max),
//    dv_max being the head's largest V descale; the row sum l still counts the unweighted
//    P~, and the epilogue multiplies O by dv_max/64/l. The lazy-rescale threshold is 2^2, so
//    the fp8 operand P~*64*dv/dv_max stays in [0, 256], inside e4m3's normal range down to
//    P~ = 2^-12.
#include "attn_device.h"
#include "attn_launch.h"

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
template <bool BF16, int D>
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
  if (p.rotate) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int idx = t * EPT + e;
      if ((p.neg[idx >> 5] >> (idx & 31)) & 1u) y[e] = -y[e];
    }
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
#pragma unroll
    for (int m = 1; m < 4; m <<= 1)
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const float o = __shfl_xor(y[e], m);
        y[e] = (t & m) ? o - y[e] : y[e] + o;
      }
    const float inv_sqrt_d = (D == 64) ? 0.125f : (D == 256) ? 0.0625f : 0.088388347648318440550f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) y[e] *= inv_sqrt_d;
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) amax = fmaxf(amax, fabsf(y[e]));
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float descale = amax > 0.f ? amax / kE4m3Max : 1.0f;

  uint32_t codes[EPT / 4];
#pragma unroll
  for (int w = 0; w < EPT / 4; ++w)
    codes[w] = cvt4_fp8(clamp448(y[4 * w] / descale), clamp448(y[4 * w + 1] / descale),
                        clamp448(y[4 * w + 2] / descale), clamp448(y[4 * w + 3] / descale));
#pragma unroll
  for (int c = 0; c < EPT / 16; ++c)
    buf_store16(r8, (uint32_t)row * H * D + t * EPT + 16 * c,
                u32x4{codes[4 * c], codes[4 * c + 1], codes[4 * c + 2], codes[4 * c + 3]});
  if (tid == 0) p.descale[((size_t)b * H + h) * nblk + blk] = descale;
}

// ---------------------------------------------------------------- fp8 attention
constexpr int kWaves = 4;
constexpr int kQW = 32;
constexpr int kBR = kWaves * kQW;
constexpr int kBC = 128;              // keys per tile
constexpr float kTau8 = 2.0f;         // lazy-rescale threshold (log2 units)
constexpr float kPScale = 64.0f;      // P~ * 64 * dv/dv_max is the fp8 PV operand
constexpr float kLog2PScale = 6.0f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// position (0..63) of key group 4*m .. 4*m+3 inside a 64-key chunk
__device__ __forceinline__ int fp8_vpos(int key) {
  const int k4 = (key >> 2) & 15;                       // key bits [5:2]
  const int p4 = ((k4 >> 1) | ((k4 & 1) << 3)) & 15;   // rotate right by one
  return (p4 << 2) | (key & 3);
}

__device__ __forceinline__ int fp8_vswz(int d) { return (d >> 1) & 7; }

template <bool OUT_BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_fp8_kernel(Fp8FwdParams p) {
  constexpr int BC = kBC;
  constexpr int KP = D + 16;                 // K8 row pitch (bytes)
  constexpr int KBYTES = BC * KP;
  constexpr int VP = BC;                     // V^T row pitch (bytes)
  constexpr int VBYTES = D * VP;
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int NKS = D / 64;
  constexpr int NKB = BC / 32;
  constexpr int NC2 = BC / 64;
  constexpr int NDB = D / 32;
  constexpr int KIT = BC * D / 16 / 256;
  constexpr int VITEMS = (BC / 4) * (D / 16);
  constexpr int VIT = (VITEMS + 255) / 256;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ float red[kWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H, N = p.N;
  const int nqt = (N + kBR - 1) / kBR;
  const int nblk = (N + 63) / 64;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const int qt = CAUSAL ? nqt - 1 - qi : qi;
  const int q0 = qt * kBR + wave * kQW;
  const int qrow = q0 + l32;

  const uint32_t row_bytes = (uint32_t)H * D;
  const size_t head_off = ((size_t)b * N * H + h) * D;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D;
  const auto rq = make_rsrc(p.q8 + head_off, nrec);
  const auto rk = make_rsrc(p.k8 + head_off, nrec);
  const auto rv = make_rsrc(p.v8 + head_off, nrec);
  const uint32_t orow = (uint32_t)H * D * 2;
  const auto ro = make_rsrc((char*)p.o + head_off * 2, (uint32_t)N * orow - (uint32_t)h * D * 2);
  const float* dq_h = p.dq + ((size_t)b * H + h) * nblk;
  const float* dk_h = p.dk + ((size_t)b * H + h) * nblk;
  const float* dv_h = p.dv + ((size_t)b * H + h) * nblk;

  // largest V descale of the head
  float dvm = 0.f;
  for (int i = tid; i < nblk; i += 256) dvm = fmaxf(dvm, dv_h[i]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) dvm = fmaxf(dvm, __shfl_xor(dvm, m));
  if (lane == 0) red[wave] = dvm;
  __syncthreads();
  dvm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  i32x8 qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const u32x4 a = buf_load16(rq, (uint32_t)qrow * row_bytes + 64 * ks + 32 * hf);
    const u32x4 c = buf_load16(rq, (uint32_t)qrow * row_bytes + 64 * ks + 32 * hf + 16);
    qreg[ks] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
  }
  const float dq_row = qrow < N ? dq_h[qrow >> 6] : 1.0f;
  const float cq = p.c * dq_row;

  const int kend = CAUSAL ? min(N, (qt + 1) * kBR) : N;
  const int nkt = (kend + BC - 1) / BC;

  u32x4 kreg[KIT];
  u32x4 vreg[VIT][4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = tid + 256 * it, c16 = i % (D / 16), kr = i / (D / 16);
      kreg[it] = buf_load16(rk, (uint32_t)(k0 + kr) * row_bytes + c16 * 16);
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int i = tid + 256 * it;
      if (VITEMS % 256 == 0 || i < VITEMS) {
        const int c16 = i % (D / 16), m = i / (D / 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) vreg[it][r] = buf_load16(rv, (uint32_t)(k0 + 4 * m + r) * row_bytes + c16 * 16);
      }
    }
  };
  auto store_tile = [&](int stage) {
    char* ks = smem + stage * STAGE;
    char* vs = ks + KBYTES;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = tid + 256 * it, c16 = i % (D / 16), kr = i / (D / 16);
      *(u32x4*)(ks + kr * KP + c16 * 16) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int i = tid + 256 * it;
      if (VITEMS % 256 == 0 || i < VITEMS) {
        const int c16 = i % (D / 16), m = i / (D / 16);
        const int pos = (4 * m & ~63) + fp8_vpos(4 * m);   // 64-key chunk + position inside it
        const int g = pos >> 4, boff = pos & 15;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = vreg[it][0][w], a1 = vreg[it][1][w], a2 = vreg[it][2][w], a3 = vreg[it][3][w];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = c16 * 16 + 4 * w + j;
            const uint32_t x = ((a0 >> (8 * j)) & 0xffu) | (((a1 >> (8 * j)) & 0xffu) << 8) |
                               (((a2 >> (8 * j)) & 0xffu) << 16) | (((a3 >> (8 * j)) & 0xffu) << 24);
            *(uint32_t*)(vs + d * VP + ((g ^ fp8_vswz(d)) & 7) * 16 + boff) = x;
          }
        }
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const bool wave_live = q0 < N;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int k0 = j * BC;
    const bool more = j + 1 < nkt;
    if (more) load_tile(k0 + BC);
    const char* ks = smem + (j & 1) * STAGE;
    const char* vs = ks + KBYTES;
    const bool skip = !wave_live || (CAUSAL && k0 > q0 + kQW - 1);
    if (!skip) {
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const char* kr = ks + (kb * 32 + l32) * KP + 64 * kk + 32 * hf;
          const u32x4 a = *(const u32x4*)kr;
          const u32x4 c = *(const u32x4*)(kr + 16);
          const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
          s[kb] = mfma_f8(av, qreg[kk], s[kb]);
        }
      }
      float coef[NC2], bias[NC2], winv[NC2];
#pragma unroll
      for (int c2 = 0; c2 < NC2; ++c2) {
        const int blk = min((k0 >> 6) + c2, nblk - 1);
        const float dv = dv_h[blk];
        coef[c2] = cq * dk_h[blk];
        const float wgt = kPScale * (dv / dvm);
        bias[c2] = fast_log2(wgt);
        winv[c2] = 1.0f / wgt;
      }
      const bool edge = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int c2 = 0; c2 < NC2; ++c2) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 2 * c2; kb < 2 * c2 + 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mt = fmaxf(mt, mx == -INFINITY ? -INFINITY : mx * coef[c2]);
      }
      mt = xhalf_max(mt);
      const float m_cand = fmaxf(m_run, mt);
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kTau8)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_cand);
        m_run = m_cand;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      i32x8 pk[NC2];
#pragma unroll
      for (int c2 = 0; c2 < NC2; ++c2) {
        const float bb = bias[c2] - m_use;
        float psum = 0.f;
#pragma unroll
        for (int kb = 2 * c2; kb < 2 * c2 + 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float e = fast_exp2(fmaf(s[kb][r], coef[c2], bb));
            if (edge) e = (s[kb][r] == -INFINITY) ? 0.f : e;
            s[kb][r] = e;
            psum += e;
          }
        l_run = fmaf(psum, winv[c2], l_run);
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const f32x16& sv = s[2 * c2 + (w >> 2)];
          const int r0 = 4 * (w & 3);
          pk[c2][w] = (int)cvt4_fp8(sv[r0], sv[r0 + 1], sv[r0 + 2], sv[r0 + 3]);
        }
      }
#pragma unroll
      for (int i = 0; i < NDB; ++i) {
        const int d = i * 32 + l32;
        const char* vrow = vs + d * VP;
        const int sw = fp8_vswz(d);
#pragma unroll
        for (int c2 = 0; c2 < NC2; ++c2) {
          const int g0 = 4 * c2 + 2 * hf;
          const u32x4 a = *(const u32x4*)(vrow + ((g0 ^ sw) & 7) * 16);
          const u32x4 c = *(const u32x4*)(vrow + (((g0 + 1) ^ sw) & 7) * 16);
          const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
          oacc[i] = mfma_f8(av, pk[c2], oacc[i]);
        }
      }
    }
    if (more) store_tile((j + 1) & 1);
    __syncthreads();
  }

  if (wave_live) {
    const float l_tot = xhalf_sum(l_run);
    const float fac = dvm / kPScale / l_tot;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        const u32x2 v = {pack2<OUT_BF16>(oacc[i][4 * rr + 0] * fac, oacc[i][4 * rr + 1] * fac),
                         pack2<OUT_BF16>(oacc[i][4 * rr + 2] * fac, oacc[i][4 * rr + 3] * fac)};
        buf_store8(ro, (uint32_t)qrow * orow + d0 * 2, v);
      }
    if (hf == 0 && qrow < N) p.lse[((size_t)b * H + h) * N + qrow] = (m_use + fast_log2(l_tot)) * kLn2;
  }
}

template <bool BF16, int D>
hipError_t launch_q(const Fp8QuantParams& p, hipStream_t s) {
  const int nblk = (p.N + 63) / 64;
  hipLaunchKernelGGL((fp8_quant_kernel<BF16, D>), dim3((unsigned)(p.B * p.H * nblk)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool OUT_BF16, int D, bool CAUSAL>
hipError_t launch_f(const Fp8FwdParams& p, hipStream_t s) {
  const int nqt = (p.N + kBR - 1) / kBR;
  hipLaunchKernelGGL((fwd_fp8_kernel<OUT_BF16, D, CAUSAL>), dim3((unsigned)(p.B * p.H * nqt)), dim3(256), 0, s, p);
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
