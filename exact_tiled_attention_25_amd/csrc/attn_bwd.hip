// Backward exact attention for gfx950, by recomputation from the stored log-sum-exp.
//
// Method (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention", Deep Dive "Backward
// warp specialization"): K_j, V_j stay put while Q_i, dO_i tiles stream past; S and P are
// recomputed from L_i, then dP, dS, dV and dK are formed, and dQ collects dS K. The page
// names the quantities only; the formulas are the softmax gradient:
//   P = exp(scale*S - L),  dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//   D_i = sum_t dO_it O_it (= sum_j P_ij dP_ij),  dK = scale dS^T Q,  dQ = scale dS K.
//
// gfx950 design. Three kernels on the caller's stream, no atomics (deterministic):
//  1. bwd_pre:  D = rowsum(dO o O) in fp32 into the workspace (HBM-bound, one pass).
//  2. bwd_dkdv: one workgroup per 128 keys of a head (4 waves x 32 keys). Each wave keeps
//     its keys' K and V in registers as MFMA B operands and its dK^T, dV^T accumulators in
//     registers; Q and dO tiles stream through a two-stage LDS ring in both row-major (for
//     S = Q K^T and dP = dO V^T) and transposed (for dV^T += dO^T P, dK^T += Q^T dS) form.
//     S and dP come out with one key per lane, so P and dS feed the next products straight
//     from the accumulators (rows reordered by swap23, matched by the transposed tiles).
//  3. bwd_dq:   one workgroup per 128 queries (like the forward): K, K^T and V tiles stream;
//     S^T = K Q^T and dP^T = V dO^T put one query per lane, so L_i and D_i are per-lane
//     scalars, and dQ^T += K^T dS^T.
// Recomputing S and dP in both 2 and 3 costs 7 matrix products instead of 5; the reported
// FLOP rate still counts 2.5 forward passes.
#include "attn_launch.h"
#include "attn_tiles.h"

namespace attn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;

template <bool BF16>
__device__ __forceinline__ void unpack2(uint32_t x, float& lo, float& hi) {
  if constexpr (BF16) {
    lo = __uint_as_float(x << 16);
    hi = __uint_as_float(x & 0xffff0000u);
  } else {
    lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
    hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  }
}

// ---------------------------------------------------------------- D = rowsum(dO o O)
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
  constexpr int TPR = D / 8;       // threads per (token, head) row, 16 bytes each
  constexpr int RPB = 256 / TPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const long nrows = (long)p.B * p.N * p.H;
  const long row = (long)blockIdx.x * RPB + tid / TPR;   // row = (b*N + n)*H + h
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 a = *(const u32x4*)((const char*)p.o + row * (D * 2) + (tid % TPR) * 16);
    const u32x4 g = *(const u32x4*)((const char*)p.dout + row * (D * 2) + (tid % TPR) * 16);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float a0, a1, g0, g1;
      unpack2<BF16>(a[w], a0, a1);
      unpack2<BF16>(g[w], g0, g1);
      acc = fmaf(a0, g0, acc);
      acc = fmaf(a1, g1, acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < nrows && tid % TPR == 0) {
    const int h = (int)(row % p.H);
    const long bn = row / p.H;
    const int n = (int)(bn % p.N), b = (int)(bn / p.N);
    p.delta[((long)b * p.H + h) * p.N + n] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV
template <int D> struct DkvCfg { static constexpr int BQ = 64; };
template <> struct DkvCfg<256> { static constexpr int BQ = 32; };

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BQ = DkvCfg<D>::BQ;
  constexpr int NQB = BQ / 32;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int BKV = kWaves * 32;
  using QT = Tile<D, BQ>;
  constexpr int OFF_DO = QT::RM_BYTES;
  constexpr int OFF_QT = 2 * QT::RM_BYTES;
  constexpr int OFF_DOT = OFF_QT + QT::T_BYTES;
  constexpr int OFF_L = OFF_DOT + QT::T_BYTES;
  constexpr int OFF_D = OFF_L + BQ * 4;
  constexpr int STAGE = OFF_D + BQ * 4;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H, N = p.N;
  const int nkvt = (N + BKV - 1) / BKV;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = work % nkvt;          // causal: low key tiles see the most queries; they go first
  const int bh = work / nkvt;
  const int h = bh % H, b = bh / H;
  const int k0 = kt * BKV;
  const int k0w = k0 + wave * 32;
  const int key = k0w + l32;

  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const size_t head_off = ((size_t)b * N * H + h) * D * 2;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D * 2;
  const auto rq = make_rsrc((const char*)p.q + head_off, nrec);
  const auto rk = make_rsrc((const char*)p.k + head_off, nrec);
  const auto rv = make_rsrc((const char*)p.v + head_off, nrec);
  const auto rdo = make_rsrc((const char*)p.dout + head_off, nrec);
  const auto rdk = make_rsrc((const char*)p.dk + head_off, nrec);
  const auto rdv = make_rsrc((const char*)p.dv + head_off, nrec);
  const float* lse_h = p.lse + ((size_t)b * H + h) * N;
  const float* del_h = p.delta + ((size_t)b * H + h) * N;

  u32x4 kreg[NKS], vreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kreg[ks] = buf_load16(rk, (uint32_t)key * row_bytes + (16 * ks + 8 * hf) * 2);
    vreg[ks] = buf_load16(rv, (uint32_t)key * row_bytes + (16 * ks + 8 * hf) * 2);
  }

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? k0 / BQ : 0;
  QT tq, tdo;
  float lval = 0.f, dval = 0.f;
  auto load_tile = [&](int qt) {
    tq.load(rq, qt * BQ, row_bytes, tid);
    tdo.load(rdo, qt * BQ, row_bytes, tid);
    if (tid < BQ) {
      const int q = qt * BQ + tid;
      lval = q < N ? lse_h[q] * kLog2e : INFINITY;   // P = exp2(s*c - inf) = 0 past the end
      dval = q < N ? del_h[q] : 0.f;
    }
  };
  auto store_tile = [&](int stage) {
    char* st = smem + stage * STAGE;
    tq.store_rowmajor(st, tid);
    tdo.store_rowmajor(st + OFF_DO, tid);
    tq.store_transposed(st + OFF_QT, tid);
    tdo.store_transposed(st + OFF_DOT, tid);
    if (tid < BQ) {
      ((float*)(st + OFF_L))[tid] = lval;
      ((float*)(st + OFF_D))[tid] = dval;
    }
  };

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }
  const bool wave_live = k0w < N;
  const float c = p.c;

  if (qt0 < nqt) {
    load_tile(qt0);
    store_tile(0);
  }
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int stage = (qt - qt0) & 1;
    const bool more = qt + 1 < nqt;
    if (more) load_tile(qt + 1);
    const char* st = smem + stage * STAGE;
    const int q0 = qt * BQ;
    const bool skip = !wave_live || (CAUSAL && q0 + BQ - 1 < k0w);
    if (!skip) {
      f32x16 s[NQB], dp[NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb] = f32x16{};
        dp[qb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          s[qb] = mfma32x16<BF16>(read_rm<D>(st, qb * 32 + l32, kk, hf), kreg[kk], s[qb]);
          dp[qb] = mfma32x16<BF16>(read_rm<D>(st + OFF_DO, qb * 32 + l32, kk, hf), vreg[kk], dp[qb]);
        }
      }
      const bool edge = CAUSAL && q0 < k0w + 31;
      const float* ls = (const float*)(st + OFF_L);
      const float* ds_ = (const float*)(st + OFF_D);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *(const f32x4*)(ls + qb * 32 + 8 * g + 4 * hf);
          const f32x4 d4 = *(const f32x4*)(ds_ + qb * 32 + 8 * g + 4 * hf);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pv = fast_exp2(fmaf(s[qb][r], c, -l4[e]));
            if (edge && key > q0 + qb * 32 + 8 * g + 4 * hf + e) pv = 0.f;
            s[qb][r] = pv;
            dp[qb][r] = pv * (dp[qb][r] - d4[e]);
          }
        }
#pragma unroll
      for (int cc = 0; cc < BQ / 16; ++cc) {
        const u32x4 ppk = pack_chunk<BF16>(s[cc >> 1], cc & 1);
        const u32x4 dspk = pack_chunk<BF16>(dp[cc >> 1], cc & 1);
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
          dvacc[i] = mfma32x16<BF16>(read_t<BQ>(st + OFF_DOT, i * 32 + l32, cc, hf), ppk, dvacc[i]);
          dkacc[i] = mfma32x16<BF16>(read_t<BQ>(st + OFF_QT, i * 32 + l32, cc, hf), dspk, dkacc[i]);
        }
      }
    }
    if (more) store_tile(stage ^ 1);
    __syncthreads();
  }

  if (wave_live) {
    const float scale = p.scale;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        const u32x2 vv = {pack2<BF16>(dvacc[i][4 * rr + 0], dvacc[i][4 * rr + 1]),
                          pack2<BF16>(dvacc[i][4 * rr + 2], dvacc[i][4 * rr + 3])};
        const u32x2 kk = {pack2<BF16>(dkacc[i][4 * rr + 0] * scale, dkacc[i][4 * rr + 1] * scale),
                          pack2<BF16>(dkacc[i][4 * rr + 2] * scale, dkacc[i][4 * rr + 3] * scale)};
        buf_store8(rdv, (uint32_t)key * row_bytes + d0 * 2, vv);
        buf_store8(rdk, (uint32_t)key * row_bytes + d0 * 2, kk);
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D> struct DqCfg { static constexpr int BC = 64; };
template <> struct DqCfg<64> { static constexpr int BC = 128; };
template <> struct DqCfg<256> { static constexpr int BC = 32; };

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
  constexpr int BC = DqCfg<D>::BC;
  constexpr int NKB = BC / 32;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int BR = kWaves * 32;
  using KT = Tile<D, BC>;
  constexpr int OFF_KT = KT::RM_BYTES;
  constexpr int OFF_V = OFF_KT + KT::T_BYTES;
  constexpr int STAGE = OFF_V + KT::RM_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H, N = p.N;
  const int nqt = (N + BR - 1) / BR;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const int qt = CAUSAL ? nqt - 1 - qi : qi;
  const int q0 = qt * BR + wave * 32;
  const int qrow = q0 + l32;

  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const size_t head_off = ((size_t)b * N * H + h) * D * 2;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D * 2;
  const auto rq = make_rsrc((const char*)p.q + head_off, nrec);
  const auto rk = make_rsrc((const char*)p.k + head_off, nrec);
  const auto rv = make_rsrc((const char*)p.v + head_off, nrec);
  const auto rdo = make_rsrc((const char*)p.dout + head_off, nrec);
  const auto rdq = make_rsrc((const char*)p.dq + head_off, nrec);

  u32x4 qreg[NKS], doreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qreg[ks] = buf_load16(rq, (uint32_t)qrow * row_bytes + (16 * ks + 8 * hf) * 2);
    doreg[ks] = buf_load16(rdo, (uint32_t)qrow * row_bytes + (16 * ks + 8 * hf) * 2);
  }
  const bool row_ok = qrow < N;
  const float lse2 = row_ok ? p.lse[((size_t)b * H + h) * N + qrow] * kLog2e : 0.f;
  const float dq_row = row_ok ? p.delta[((size_t)b * H + h) * N + qrow] : 0.f;

  const int kend = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nkt = (kend + BC - 1) / BC;
  KT tk, tv;
  auto load_tile = [&](int k0) {
    tk.load(rk, k0, row_bytes, tid);
    tv.load(rv, k0, row_bytes, tid);
  };
  auto store_tile = [&](int stage) {
    char* st = smem + stage * STAGE;
    tk.store_rowmajor(st, tid);
    tk.store_transposed(st + OFF_KT, tid);
    tv.store_rowmajor(st + OFF_V, tid);
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};
  const bool wave_live = q0 < N;
  const float c = p.c;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int j = 0; j < nkt; ++j) {
    const int k0 = j * BC;
    const bool more = j + 1 < nkt;
    if (more) load_tile(k0 + BC);
    const char* st = smem + (j & 1) * STAGE;
    const bool skip = !wave_live || (CAUSAL && k0 > q0 + 31);
    if (!skip) {
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          s[kb] = mfma32x16<BF16>(read_rm<D>(st, kb * 32 + l32, kk, hf), qreg[kk], s[kb]);
          dp[kb] = mfma32x16<BF16>(read_rm<D>(st + OFF_V, kb * 32 + l32, kk, hf), doreg[kk], dp[kb]);
        }
      }
      const bool edge = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = fast_exp2(fmaf(s[kb][r], c, -lse2));
          if (edge) {
            const int kidx = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (kidx >= N || (CAUSAL && kidx > qrow)) pv = 0.f;
          }
          s[kb][r] = pv * (dp[kb][r] - dq_row);
        }
#pragma unroll
      for (int cc = 0; cc < BC / 16; ++cc) {
        const u32x4 dspk = pack_chunk<BF16>(s[cc >> 1], cc & 1);
#pragma unroll
        for (int i = 0; i < NDB; ++i)
          dqacc[i] = mfma32x16<BF16>(read_t<BC>(st + OFF_KT, i * 32 + l32, cc, hf), dspk, dqacc[i]);
      }
    }
    if (more) store_tile((j + 1) & 1);
    __syncthreads();
  }

  if (wave_live) {
    const float scale = p.scale;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        const u32x2 vv = {pack2<BF16>(dqacc[i][4 * rr + 0] * scale, dqacc[i][4 * rr + 1] * scale),
                          pack2<BF16>(dqacc[i][4 * rr + 2] * scale, dqacc[i][4 * rr + 3] * scale)};
        buf_store8(rdq, (uint32_t)qrow * row_bytes + d0 * 2, vv);
      }
  }
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_t(const BwdParams& p, hipStream_t s) {
  const long nrows = (long)p.B * p.N * p.H;
  const int rpb = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<BF16, D>), dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkvt = (p.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, CAUSAL>), dim3((unsigned)(p.B * p.H * nkvt)), dim3(256), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nqt = (p.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, CAUSAL>), dim3((unsigned)(p.B * p.H * nqt)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_c(bool causal, const BwdParams& p, hipStream_t s) {
  return causal ? launch_t<BF16, D, true>(p, s) : launch_t<BF16, D, false>(p, s);
}

template <bool BF16>
hipError_t launch_d(int d, bool causal, const BwdParams& p, hipStream_t s) {
  switch (d) {
    case 64: return launch_c<BF16, 64>(causal, p, s);
    case 128: return launch_c<BF16, 128>(causal, p, s);
    case 256: return launch_c<BF16, 256>(causal, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_bwd(bool bf16, int d, bool causal, const BwdParams& p, hipStream_t s) {
  return bf16 ? launch_d<true>(d, causal, p, s) : launch_d<false>(d, causal, p, s);
}

}  // namespace attn
