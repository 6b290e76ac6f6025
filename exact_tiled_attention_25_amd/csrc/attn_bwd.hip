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
//  1. bwd_pre:  D = rowsum(dO o O) in fp32 into the workspace, next to L log2 e (HBM-bound,
//     one pass): the pair of a row is one 8-byte word, so the kernels below take a tile's
//     L and D in one piece.
//  2. bwd_dkdv: one workgroup per 128 keys of a key/value head (4 waves x 32 keys); with
//     grouped key/value heads it visits the Q tiles of every query head of the group, so
//     dK and dV are summed in registers (no atomics). Each wave keeps
//     its keys' K and V in registers as MFMA B operands and its dK^T, dV^T accumulators in
//     registers; Q and dO tiles stream through a three-stage LDS ring in both row-major (for
//     S = Q K^T and dP = dO V^T) and transposed (for dV^T += dO^T P, dK^T += Q^T dS) form.
//     S and dP come out with one key per lane, so P and dS feed the next products straight
//     from the accumulators (rows reordered by swap23, matched by the transposed tiles).
//  3. bwd_dq:   one workgroup per 128 queries (like the forward): K, K^T and V tiles stream;
//     S^T = K Q^T and dP^T = V dO^T put one query per lane, so L_i and D_i are per-lane
//     scalars, and dQ^T += K^T dS^T.
// Recomputing S and dP in both 2 and 3 costs 7 matrix products instead of 5; the reported
// FLOP rate still counts 2.5 forward passes.
#include <type_traits>

#include "attn_launch.h"
#include "attn_lds.h"

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
  // rows (token, head): (b*N + n)*H + h, or t*H + h of the packed variable-length tokens
  const long nrows = p.cu ? (long)p.T * p.H : (long)p.B * p.N * p.H;
  const long row = (long)blockIdx.x * RPB + tid / TPR;
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
    long i;
    if (p.cu) {
      i = (long)h * p.T + bn;
    } else {
      const int n = (int)(bn % p.N), b = (int)(bn / p.N);
      i = ((long)b * p.H + h) * p.N + n;
    }
    ((float2*)p.stats)[i] = float2{p.lse[i] * kLog2e, acc};
  }
}

// ---------------------------------------------------------------- dK, dV
// KV-outer: 4 waves x 32 keys per workgroup. Each wave keeps its keys' K and V as MFMA B
// operands in registers and its dK^T, dV^T accumulators in registers. Q and dO tiles of BQ
// queries and the tile's (L log2 e, D) pairs arrive by DMA in a three-stage LDS ring (read
// as rows for S = Q K^T and dP = dO V^T, read transposed for dV^T += dO^T P and dK^T +=
// Q^T dS). A tile's DMA is issued two tiles ahead of its use: one tile of MFMA work
// (about 1 us) does not cover an HBM round trip under load. S and dP put one key per lane, so P and
// dS feed the next products straight from the accumulators. The 64-query tile is worked
// in two 32-query halves so that the VALU work of one half runs under the other's MFMAs:
// scores(0) | scores(1) + softmax(0) | update(0) + softmax(1) | update(1).
// Step schedule of one Q tile in the dK/dV kernel (NQB 32-query blocks; SC score steps and
// UP update steps per block): softmax elements per step (ES during the scores of block 1,
// EU during the update of block 0) and the register ring that holds the L and D values of
// query group (qb, m) from its LDS read, LPF steps ahead of its first use, to its last use.
template <int NQB, int SC, int UP>
struct DkvSched {
  static constexpr int ES = (16 + SC - 1) / SC, EU = (16 + UP - 1) / UP;
  static constexpr int LPF = 4;
  static constexpr int LRS = NQB == 1 ? 4 : ES >= 2 ? 3 : 2;
  static constexpr int use(int qb, int m, int last) {   // first (last = 0) or last step using the group
    return NQB == 1 ? SC : qb == 0 ? SC + (4 * m + 3 * last) / ES : 2 * SC + (4 * m + 3 * last) / EU;
  }
  static constexpr int load(int qb, int m) { return use(qb, m, 0) - LPF; }
  static constexpr bool ring_ok() {   // a slot is reloaded only after the last use of its group
    for (int a = 0; a < 4 * NQB; ++a)
      for (int b = a + 1; b < 4 * NQB; ++b)
        if (a % LRS == b % LRS && load(b / 4, b % 4) <= use(a / 4, a % 4, 1)) return false;
    return load(0, 0) >= 0;
  }
};

template <int D> struct DkvCfg { static constexpr int BQ = 64, OCC = 1; };
template <> struct DkvCfg<64> { static constexpr int BQ = 64, OCC = 2; };
template <> struct DkvCfg<256> { static constexpr int BQ = 32, OCC = 1; };

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256, DkvCfg<D>::OCC) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BQ = DkvCfg<D>::BQ;
  constexpr int NQB = BQ / 32;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int BKV = kWaves * 32;
  // d <= 128: unpadded Q/dO tiles with the chunk swizzle (conflict-free row and transpose
  // reads); d = 256 (no registers to spare for the read offsets): padded pitch 2d + 48.
  constexpr int SWZ = D <= 128 ? D : 0;
  constexpr int QP = SWZ ? 2 * D : rt_pitch<D>();
  using QPlan = DmaPlan<D, BQ, QP, kWaves>;
  constexpr int TB = QPlan::BYTES;
  // Stage: Q tile, dO tile, then one 256-byte slot per wave for the (L log2 e, D) pairs of
  // tile rows 16w .. 16w+15 (first half; the second half takes the DMA's idle lanes).
  constexpr int NSTAGE = 3;
  constexpr int OFF_DO = TB, OFF_LD = 2 * TB;
  constexpr int STAGE = 2 * TB + kWaves * 256;
  static_assert(16 * kWaves >= BQ, "one L/D slot per 16 rows");
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps loop control scalar
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H, Hkv = p.Hkv, G = H / Hkv;
  const int nkvt = (p.N + BKV - 1) / BKV;   // p.N: the (longest) sequence length
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int kt = work % nkvt;          // causal: low key tiles see the most queries; they go first
  const int bh = spread_pair(work / nkvt, p.B * Hkv, p.cu != nullptr);
  const int kvh = bh % Hkv, b = bh / Hkv;   // key/value head; its query heads are kvh*G .. +G-1
  const SeqView sv = seq_view(p.cu, b, p.N, p.T);
  const int N = sv.len;
  if (kt * BKV >= N) return;   // a shorter sequence of a variable-length batch: nothing here
  const int k0w = kt * BKV + wave * 32;
  const int key = k0w + l32;

  // K, V, dK, dV: [B][N][Hkv][D]; Q, dO: [B][N][H][D]; L, D: [B][H][N]
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const size_t kv_head_off = ((size_t)sv.start * Hkv + kvh) * D * 2;
  const uint32_t kv_nrec = (uint32_t)N * kv_row_bytes - (uint32_t)kvh * D * 2;
  const auto rk = make_rsrc((const char*)p.k + kv_head_off, kv_nrec);
  const auto rv = make_rsrc((const char*)p.v + kv_head_off, kv_nrec);
  const auto rdk = make_rsrc((const char*)p.dk + kv_head_off, kv_nrec);
  const auto rdv = make_rsrc((const char*)p.dv + kv_head_off, kv_nrec);
  const uint32_t row_bytes = (uint32_t)H * D * 2;

  const int nqt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? (kt * BKV) / BQ : 0;
  // The workgroup visits query tiles qt0 .. nqt-1 of each of its G query heads. Causal: the
  // tiles before qe reach this workgroup's keys and need the mask. Order (u numbers it): the
  // masked tiles of every head, then the plain tiles of every head; two straight-line loops,
  // as dK and dV are sums in any order.
  // Positions advance by compares only (a division here would be scheduled into the tile
  // body, where every register is taken).
  const int qe = CAUSAL ? max(qt0, min(nqt, (kt * BKV + BKV - 1 + BQ - 1) / BQ)) : qt0;
  const int UE = G * (qe - qt0), NU = G * (nqt - qt0);
  struct Pos { int g, qt; };   // query head kvh*G + g, query tile qt
  auto first_pos = [&]() { return qe > qt0 ? Pos{0, qt0} : Pos{0, qe}; };
  auto next_pos = [&](Pos q) {
    if (q.qt < qe) {   // masked tiles: qt0 .. qe-1 of each head, then the first plain tile
      if (q.qt + 1 < qe) return Pos{q.g, q.qt + 1};
      return q.g + 1 < G ? Pos{q.g + 1, qt0} : Pos{0, qe};
    }
    return q.qt + 1 < nqt ? Pos{q.g, q.qt + 1} : Pos{q.g + 1, qe};
  };
  uint32_t qvoff[QPlan::NPW];
  dma_init<QPlan, kWaves, SWZ>(qvoff, row_bytes, wave, lane);
  // L/D DMA (4 bytes a lane): wave w brings the 32 words of rows 16w .. 16w+15 with lanes
  // 0-31; lanes 32-63, and rows past the tile, are pointed past the buffer's end.
  const uint32_t ld_voff = (lane < 32 && 16 * wave < BQ) ? (uint32_t)(32 * wave + lane) * 4 : 0x80000000u;
  // DMA instructions this wave issues per tile (Q, dO, L/D), and the most of any wave
  const int dma_per_tile = 2 * dma_count<QPlan, kWaves>(wave) + 1;
  constexpr int MAX_PER_TILE = 2 * QPlan::NPW + 1;
  auto fetch_into = [&](Pos ps, char* st) {
    // the tile position is the same in every lane; the compiler cannot tell through the
    // loop-carried position (it would wrap each DMA instruction in a loop over lanes)
    const int qt = (int)uniform((uint32_t)ps.qt), hq = kvh * G + (int)uniform((uint32_t)ps.g);
    const size_t qh_off = ((size_t)sv.start * H + hq) * D * 2;
    const uint32_t q_nrec = (uint32_t)N * row_bytes - (uint32_t)hq * D * 2;
    dma_issue<QPlan, kWaves>(qvoff, st, (const char*)p.q + qh_off, qt * BQ, row_bytes, q_nrec, wave);
    dma_issue<QPlan, kWaves>(qvoff, st + OFF_DO, (const char*)p.dout + qh_off, qt * BQ, row_bytes, q_nrec, wave);
    // Rows past the end arrive as zeros: L = D = 0 there, and with their Q and dO rows zero
    // too, P = 1 multiplies zeros (no contribution to dK or dV).
    const size_t lrow = stat_row(p.cu, p.T, b, H, hq, sv) + (size_t)qt * BQ;
    const auto rl = make_rsrc(p.stats + 2 * lrow, (uint32_t)(N - qt * BQ) * 8);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)(st + OFF_LD + wave * 256), 4, ld_voff, 0, 0, 0);
  };

  u32x4 kreg[NKS], vreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kreg[ks] = buf_load16(rk, (uint32_t)key * kv_row_bytes + (16 * ks + 8 * hf) * 2);
    vreg[ks] = buf_load16(rv, (uint32_t)key * kv_row_bytes + (16 * ks + 8 * hf) * 2);
  }
  // the first two tiles; the loop issues each next one two tiles ahead
  Pos pos0 = first_pos(), pos1 = next_pos(pos0), pos2 = next_pos(pos1);   // tiles u, u+1, u+2
  if (NU > 0) fetch_into(pos0, smem);
  if (NU > 1) fetch_into(pos1, smem + STAGE);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {   // waited for here, not inside the tile loop
    settle(kreg[ks]);
    settle(vreg[ks]);
  }
  // One wave per SIMD (512 registers): every MFMA accumulator (dK, dV for the whole kernel,
  // S and dP per block) lives in AGPRs; K, V and everything the VALU writes in VGPRs.
  // Without the hint the allocator shares AGPRs between S/dP and dK/dV and copies the
  // evicted accumulators back and forth every tile.
  constexpr bool PIN = DkvCfg<D>::OCC == 1;
  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }
  const bool wave_live = k0w < N;
  const float c = p.c;
  const int row_q = row_lane_off<QP>(lane), tr_q = tr_lane_off<QP>(lane);
  int srow[SWZ ? D / 16 : 1], str_[2][SWZ ? D / 32 : 1];
  if constexpr (SWZ != 0) swz_offsets<D>(lane, srow, str_);

  wait_dma_keep_rt<MAX_PER_TILE>(NU > 1 ? dma_per_tile : 0);   // tile 0 landed; tile 1 may still fly
  __syncthreads();

  auto tile = [&](const char* st, int q0, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const char* qr = st + row_q;
    const char* qtr = st + tr_q;
    const char* dr = st + OFF_DO + row_q;
    const char* dtr = st + OFF_DO + tr_q;
    const char* ldp = st + OFF_LD + 32 * hf;   // this lane half's 4-row groups within a slot
    f32x16 s[NQB], dp[NQB];
    u32x4 ppk[2 * NQB], dspk[2 * NQB];
    // L and D of query group (qb, m) = queries 8m + 4hf .. +3 of block qb, read from LDS
    // into a small register ring LPF steps before the softmax step that first needs them
    // (reading them at the point of use would stall on the whole LDS queue every time).
    constexpr int SC = 2 * NKS;        // MFMAs of scores(qb): S and dP alternate
    constexpr int UP = 2 * 2 * NDB;    // MFMAs of update(qb): dV and dK alternate over 2 chunks x NDB blocks
    using Sched = DkvSched<NQB, SC, UP>;
    static_assert(Sched::ring_ok(), "L/D ring slot reused while live");
    constexpr int ES = Sched::ES, EU = Sched::EU, LRS = Sched::LRS;
    f32x4 lring[LRS], dring[LRS];
    auto load_grp = [&](int qb, int m) {
      // rows r0 .. r0+3, r0 = 32 qb + 8 m + 4 hf: slot r0/16, (L, D) pairs from (r0 % 16) * 8
      const int c0 = qb * 32 + 8 * m;
      const char* a = ldp + (c0 >> 4) * 256 + (c0 & 15) * 8;
      const f32x4 x = *(const f32x4*)a, y = *(const f32x4*)(a + 16);
      lring[(4 * qb + m) % LRS] = f32x4{x[0], x[2], y[0], y[2]};
      dring[(4 * qb + m) % LRS] = f32x4{x[1], x[3], y[1], y[3]};
    };
    // softmax(qb) element r: P and dS of query 8*(r/4) + 4*hf + r%4 of block qb
    auto sm_elem = [&](int qb, int r) {
      const f32x4& l4 = lring[(4 * qb + (r >> 2)) % LRS];
      const f32x4& d4 = dring[(4 * qb + (r >> 2)) % LRS];
      float pv = fast_exp2(fmaf(s[qb][r], c, -l4[r & 3]));
      if constexpr (EDGE) {
        if (CAUSAL && key > q0 + qb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)) pv = 0.f;
      }
      s[qb][r] = pv;
      dp[qb][r] = pv * (dp[qb][r] - d4[r & 3]);
      if ((r & 7) == 7) {
        const int b8 = r - 7;
        ppk[2 * qb + (r >> 3)] = u32x4{pack2<BF16>(s[qb][b8], s[qb][b8 + 1]), pack2<BF16>(s[qb][b8 + 2], s[qb][b8 + 3]),
                                       pack2<BF16>(s[qb][b8 + 4], s[qb][b8 + 5]), pack2<BF16>(s[qb][b8 + 6], s[qb][b8 + 7])};
        dspk[2 * qb + (r >> 3)] = u32x4{pack2<BF16>(dp[qb][b8], dp[qb][b8 + 1]), pack2<BF16>(dp[qb][b8 + 2], dp[qb][b8 + 3]),
                                        pack2<BF16>(dp[qb][b8 + 4], dp[qb][b8 + 5]), pack2<BF16>(dp[qb][b8 + 6], dp[qb][b8 + 7])};
      }
    };
    // The tile is one static sequence of MFMA steps: scores(0), scores(1), update(0), update(1)
    // (NQB = 2) or scores(0), update(0) (NQB = 1). The LDS operand of step g is read PF
    // steps ahead; the softmax of block 0 rides on scores(1), that of block 1 on update(0).
    constexpr int T = NQB * (SC + UP);
    constexpr int PF = 4;
    auto operand = [&](int g) -> u32x4 {
      if (g < NQB * SC) {
        const int qb = g / SC, t = g % SC, kk = t >> 1;
        if constexpr (SWZ != 0) return lds_read16(st + ((t & 1) ? OFF_DO : 0) + srow[kk] + qb * 32 * QP);
        return (t & 1) ? lds_row<QP>(dr, qb, kk) : lds_row<QP>(qr, qb, kk);
      }
      const int qb = (g - NQB * SC) / UP, t = (g - NQB * SC) % UP;
      const int cc = 2 * qb + t / (2 * NDB), i = (t >> 1) % NDB;
      if constexpr (SWZ != 0) {
        const char* base = st + ((t & 1) ? 0 : OFF_DO) + cc * 16 * QP;
        return lds_tr_pair(base + str_[0][i], base + str_[1][i]);
      }
      return (t & 1) ? lds_tr<QP>(qtr, cc, i) : lds_tr<QP>(dtr, cc, i);
    };
    auto mfma_step = [&](int g, const u32x4& op) {
      if (g < NQB * SC) {
        const int qb = g / SC, t = g % SC, kk = t >> 1;
        if (t & 1) {
          dp[qb] = mfma32x16<BF16>(op, vreg[kk], kk == 0 ? f32x16{} : dp[qb]);
          if constexpr (PIN) pin_acc(dp[qb]);
        } else {
          s[qb] = mfma32x16<BF16>(op, kreg[kk], kk == 0 ? f32x16{} : s[qb]);
          if constexpr (PIN) pin_acc(s[qb]);
        }

      } else {
        const int qb = (g - NQB * SC) / UP, t = (g - NQB * SC) % UP;
        const int cc = 2 * qb + t / (2 * NDB), i = (t >> 1) % NDB;
        if (t & 1) {
          dkacc[i] = mfma32x16<BF16>(op, dspk[cc], dkacc[i]);
          if constexpr (PIN) pin_acc(dkacc[i]);
        } else {
          dvacc[i] = mfma32x16<BF16>(op, ppk[cc], dvacc[i]);
          if constexpr (PIN) pin_acc(dvacc[i]);
        }
      }
    };
    u32x4 ring[PF + 1];
    __builtin_amdgcn_sched_barrier(0);
    static_for<PF>([&](auto gc) { ring[decltype(gc)::value] = operand(decltype(gc)::value); });
    static_for<T>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      static_for<NQB * 4>([&](auto mc) {
        constexpr int qb = decltype(mc)::value / 4, m = decltype(mc)::value % 4;
        if constexpr (Sched::load(qb, m) == g) load_grp(qb, m);
      });
      if constexpr (NQB == 1 && g == SC) {
        // single block: its softmax sits between the score and update steps
        static_for<16>([&](auto rc) { sm_elem(0, decltype(rc)::value); });
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (g + PF < T) ring[(g + PF) % (PF + 1)] = operand(g + PF);
      mfma_step(g, ring[g % (PF + 1)]);
      if constexpr (NQB == 2) {
        if constexpr (g >= SC && g < 2 * SC) {
          static_for<ES>([&](auto uc) {
            constexpr int r = ES * (g - SC) + decltype(uc)::value;
            if constexpr (r < 16) sm_elem(0, r);
          });
        } else if constexpr (g >= 2 * SC && g < 2 * SC + UP) {
          static_for<EU>([&](auto uc) {
            constexpr int r = EU * (g - 2 * SC) + decltype(uc)::value;
            if constexpr (r < 16) sm_elem(1, r);
          });
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  auto pin_all = [&]() {
    if constexpr (PIN) {
#pragma unroll
      for (int a = 0; a < NDB; ++a) {
        pin_acc(dkacc[a]);
        pin_acc(dvacc[a]);
      }
    }
  };
  // Causal: the first tiles (those that reach a key of this workgroup) need the mask, and
  // waves whose keys all follow the tile skip it; the rest need neither. Two loops keep each
  // loop body straight-line (one tile form, no skip branch), so the accumulators stay put.
  // Waves past the end of the sequence compute on zero-filled K, V and store nothing.
  // One Q tile: DMA of tile u + 2 into stage `nxt` (the stage tile u - 1 used) and the math
  // on stage `cur`. The stages are distinct, and saying so (restrict) lets the compiler see
  // that the tile's LDS reads cannot alias the DMA in flight: otherwise it waits for that
  // DMA before the first transpose read of the tile.
  auto body = [&](int u, char* __restrict__ nxt, const char* __restrict__ cur, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    if (u + 2 < NU) fetch_into(pos2, nxt);
    const int q0 = pos0.qt * BQ;
    if constexpr (EDGE) {
      if (wave_live && q0 + BQ - 1 >= k0w) tile(cur, q0, std::true_type{});
    } else {
      tile(cur, q0, std::false_type{});
    }
  };
  int sc = 0;   // stage of tile u (u mod 3)
  auto step = [&](int u, auto edge_tag) {
    pin_all();
    const int cur = __builtin_amdgcn_readfirstlane(sc * STAGE);
    const int nxt = __builtin_amdgcn_readfirstlane((sc == 0 ? NSTAGE - 1 : sc - 1) * STAGE);
    body(u, smem + nxt, smem + cur, edge_tag);
    pos0 = pos1;
    pos1 = pos2;
    pos2 = next_pos(pos2);
    // tile u + 1 has landed (in every wave, after the barrier); tile u + 2 may still fly
    wait_dma_keep_rt<MAX_PER_TILE>(u + 2 < NU ? dma_per_tile : 0);
    ring_barrier();
    sc = sc == NSTAGE - 1 ? 0 : sc + 1;
    pin_all();
  };
  int u = 0;
  if constexpr (CAUSAL) {
    for (; u < UE; ++u) step(u, std::true_type{});
  }
  for (; u < NU; ++u) step(u, std::false_type{});

  // dV, then dK, leave through the ring's LDS, each wave in its own area (the last step
  // waited for every DMA and passed a barrier after every wave's last operand read).
  using OStage = RowStage<2 * D>;
  static_assert(kWaves * OStage::BYTES <= (int)sizeof(smem), "dK/dV staging fits the ring");
  if (wave_live) {
    const float scale = p.scale;
    char* ost = smem + wave * OStage::BYTES;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        OStage::put(ost, l32, d0 * 2, u32x2{pack2<BF16>(dvacc[i][4 * rr + 0], dvacc[i][4 * rr + 1]),
                                            pack2<BF16>(dvacc[i][4 * rr + 2], dvacc[i][4 * rr + 3])});
      }
    OStage::store(ost, rdv, (uint32_t)k0w, kv_row_bytes, 0, lane);
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        OStage::put(ost, l32, d0 * 2, u32x2{pack2<BF16>(dkacc[i][4 * rr + 0] * scale, dkacc[i][4 * rr + 1] * scale),
                                            pack2<BF16>(dkacc[i][4 * rr + 2] * scale, dkacc[i][4 * rr + 3] * scale)});
      }
    OStage::store(ost, rdk, (uint32_t)k0w, kv_row_bytes, 0, lane);
  }
}

// ---------------------------------------------------------------- dQ
// Q-outer, like the forward: 4 waves x 32 query rows; K and V tiles arrive by DMA in a
// two-stage LDS ring (padded rows). Per tile, three phases with their instructions
// interleaved: S^T = K Q^T (K rows); dP^T = V dO^T (V rows) with P = exp2(s*c - L) on the
// VALU underneath; dQ^T += K^T dS^T (K read transposed) with dS = P o (dP - D) of the next
// 16-key chunk computed underneath. Tiles that touch the diagonal or the ragged end zero
// the masked P explicitly.
template <int D> struct DqCfg { static constexpr int BC = 64, OCC = 2, WAVES = 4; };
template <> struct DqCfg<256> { static constexpr int BC = 64, OCC = 1, WAVES = 4; };   // 64 keys: 15% faster than 32 at d = 256

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(64 * DqCfg<D>::WAVES, DqCfg<D>::OCC) void bwd_dq_kernel(BwdParams p) {
  constexpr int kWaves = DqCfg<D>::WAVES;
  constexpr int BC = DqCfg<D>::BC;
  constexpr int NKB = BC / 32;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int BR = kWaves * 32;
  // K tiles are read both as rows and transposed: unpadded with the chunk swizzle at d <= 128
  // (padded pitch 2d + 48 at d = 256); V tiles only as rows.
  constexpr int SWZ = D <= 128 ? D : 0;
  constexpr int KP = SWZ ? 2 * D : rt_pitch<D>(), VP = k_pitch<D>();
  using KPlan = DmaPlan<D, BC, KP, kWaves>;
  using VPlan = DmaPlan<D, BC, VP, kWaves>;
  constexpr int KB = KPlan::BYTES, VB = VPlan::BYTES, STAGE = KB + VB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  // the DMA's LDS base depends on the wave index: give it a provably uniform copy (with the
  // plain index the compiler wraps each DMA instruction in a loop over lanes; making the
  // wave index itself scalar everywhere changes the register allocation and spills)
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H;
  const int nqt = (p.N + BR - 1) / BR;   // p.N: the (longest) sequence length
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = work % nqt;
  const int bh = spread_pair(work / nqt, p.B * H, p.cu != nullptr);
  const int h = bh % H, b = bh / H;
  const SeqView sv = seq_view(p.cu, b, p.N, p.T);
  const int N = sv.len;
  const int qt = CAUSAL ? nqt - 1 - qi : qi;
  if (qt * BR >= N) return;   // a shorter sequence of a variable-length batch: nothing here
  const int q0 = qt * BR + wave * 32;
  const int qrow = q0 + l32;

  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const size_t head_off = ((size_t)sv.start * H + h) * D * 2;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D * 2;
  const auto rq = make_rsrc((const char*)p.q + head_off, nrec);
  const auto rdo = make_rsrc((const char*)p.dout + head_off, nrec);
  const auto rdq = make_rsrc((const char*)p.dq + head_off, nrec);
  // K and V: [B][N][Hkv][D], key/value head h / (H / Hkv)
  const int Hkv = p.Hkv, kvh = h / (H / Hkv);
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const size_t kv_head_off = ((size_t)sv.start * Hkv + kvh) * D * 2;
  const uint32_t kv_nrec = (uint32_t)N * kv_row_bytes - (uint32_t)kvh * D * 2;
  const char* kbase = (const char*)p.k + kv_head_off;
  const char* vbase = (const char*)p.v + kv_head_off;

  const int kend = CAUSAL ? min(N, (qt + 1) * BR) : N;
  const int nkt = (kend + BC - 1) / BC;
  const int nkt_w = q0 >= N ? 0 : CAUSAL ? min(nkt, (q0 + 31) / BC + 1) : nkt;
  uint32_t kvoff[KPlan::NPW], vvoff[VPlan::NPW];
  dma_init<KPlan, kWaves, SWZ>(kvoff, kv_row_bytes, wave, lane);
  dma_init<VPlan, kWaves>(vvoff, kv_row_bytes, wave, lane);
  auto fetch_into = [&](int j, char* st) {
    dma_issue<KPlan, kWaves>(kvoff, st, kbase, j * BC, kv_row_bytes, kv_nrec, wave_u);
    dma_issue<VPlan, kWaves>(vvoff, st + KB, vbase, j * BC, kv_row_bytes, kv_nrec, wave_u);
  };
  fetch_into(0, smem);

  u32x4 qreg[NKS], doreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qreg[ks] = buf_load16(rq, (uint32_t)qrow * row_bytes + (16 * ks + 8 * hf) * 2);
    doreg[ks] = buf_load16(rdo, (uint32_t)qrow * row_bytes + (16 * ks + 8 * hf) * 2);
  }
  const bool row_ok = qrow < N;
  const size_t stat_i = stat_row(p.cu, p.T, b, H, h, sv) + qrow;
  const float2 lrow = row_ok ? ((const float2*)p.stats)[stat_i] : float2{0.f, 0.f};
  const float lse2 = lrow.x, drow = lrow.y;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {   // waited for here, not inside the tile loop
    settle(qreg[ks]);
    settle(doreg[ks]);
  }
  settle(lse2);
  settle(drow);

  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};
  const float c = p.c;
  const int row_k = row_lane_off<KP>(lane), tr_k = tr_lane_off<KP>(lane), row_v = row_lane_off<VP>(lane);
  int srow[SWZ ? D / 16 : 1], str_[2][SWZ ? D / 32 : 1];
  if constexpr (SWZ != 0) swz_offsets<D>(lane, srow, str_);
  auto k_row = [&](const char* st, int kb, int kk) -> u32x4 {
    if constexpr (SWZ != 0) return lds_read16(st + srow[kk] + kb * 32 * KP);
    return lds_row<KP>(st + row_k, kb, kk);
  };
  auto k_tr = [&](const char* st, int c, int i) -> u32x4 {
    if constexpr (SWZ != 0) return lds_tr_pair(st + c * 16 * KP + str_[0][i], st + c * 16 * KP + str_[1][i]);
    return lds_tr<KP>(st + tr_k, c, i);
  };

  wait_dma();
  __syncthreads();

  constexpr int S1 = NKB * NKS;            // MFMAs per score product
  constexpr int EPS = 16 * NKB / S1;       // exponentials per dP step
  constexpr int PF = 3;
  auto tile = [&](int j, const char* st, auto edge_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    const char* vr = st + KB + row_v;
    const int k0 = j * BC;
    f32x16 s[NKB], dp[NKB];
    u32x4 op[S1];
    // phase 1: S^T = K Q^T
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < PF; ++t) op[t] = k_row(st, t % NKB, t / NKB);
#pragma unroll
    for (int t = 0; t < S1; ++t) {
      if (t + PF < S1) op[t + PF] = k_row(st, (t + PF) % NKB, (t + PF) / NKB);
      const int kb = t % NKB, kk = t / NKB;
      s[kb] = mfma32x16<BF16>(op[t], qreg[kk], kk == 0 ? f32x16{} : s[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase 2: dP^T = V dO^T, with P on the VALU
#pragma unroll
    for (int t = 0; t < PF; ++t) op[t] = lds_row<VP>(vr, t % NKB, t / NKB);
#pragma unroll
    for (int t = 0; t < S1; ++t) {
      if (t + PF < S1) op[t + PF] = lds_row<VP>(vr, (t + PF) % NKB, (t + PF) / NKB);
      const int kb = t % NKB, kk = t / NKB;
      dp[kb] = mfma32x16<BF16>(op[t], doreg[kk], kk == 0 ? f32x16{} : dp[kb]);
#pragma unroll
      for (int u = 0; u < EPS; ++u) {
        const int i = EPS * t + u;
        float pv = fast_exp2(fmaf(s[i >> 4][i & 15], c, -lse2));
        if constexpr (EDGE) {
          const int key = k0 + (i >> 4) * 32 + 8 * ((i & 15) >> 2) + 4 * hf + (i & 3);
          if (key >= N || (CAUSAL && key > qrow)) pv = 0.f;
        }
        s[i >> 4][i & 15] = pv;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase 3: dQ^T += K^T dS^T, dS of chunk c+1 computed under chunk c's MFMAs
    u32x4 dspk[BC / 16];
    auto ds_chunk = [&](int cc) {
      const int kb = cc >> 1, base = (cc & 1) * 8;
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = s[kb][base + t] * (dp[kb][base + t] - drow);
      dspk[cc] = u32x4{pack2<BF16>(v[0], v[1]), pack2<BF16>(v[2], v[3]), pack2<BF16>(v[4], v[5]), pack2<BF16>(v[6], v[7])};
    };
    u32x4 kop[BC / 16 * NDB];
#pragma unroll
    for (int t = 0; t < PF; ++t) kop[t] = k_tr(st, t / NDB, t % NDB);
    ds_chunk(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < BC / 16 * NDB; ++t) {
      if (t + PF < BC / 16 * NDB) kop[t + PF] = k_tr(st, (t + PF) / NDB, (t + PF) % NDB);
      const int cc = t / NDB, i = t % NDB;
      dqacc[i] = mfma32x16<BF16>(kop[t], dspk[cc], dqacc[i]);
      if (i == NDB - 1 && cc + 1 < BC / 16) ds_chunk(cc + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // DMA of the next tile into stage `nxt` and the math on stage `cur`: distinct stages,
  // passed as restrict pointers so that the tile's LDS reads are not made to wait for the
  // DMA in flight (the wait at the end of the iteration covers the next tile).
  auto body = [&](int j, char* __restrict__ nxt, const char* __restrict__ cur) {
    if (j + 1 < nkt) fetch_into(j + 1, nxt);
    if (j < nkt_w) {
      const int k0 = j * BC;
      if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0)) tile(j, cur, std::true_type{});
      else tile(j, cur, std::false_type{});
    }
  };
  for (int j = 0; j < nkt; ++j) {
    const int cur = (j & 1) * STAGE;
    body(j, smem + (STAGE - cur), smem + cur);
    wait_dma();
    __syncthreads();
  }

  // dQ leaves through the ring's LDS, each wave in its own area (the loop ended with a DMA
  // wait and a barrier).
  using OStage = RowStage<2 * D>;
  static_assert(kWaves * OStage::BYTES <= (int)sizeof(smem), "dQ staging fits the ring");
  if (nkt_w > 0) {
    const float scale = p.scale;
    char* ost = smem + wave * OStage::BYTES;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        OStage::put(ost, l32, d0 * 2, u32x2{pack2<BF16>(dqacc[i][4 * rr + 0] * scale, dqacc[i][4 * rr + 1] * scale),
                                            pack2<BF16>(dqacc[i][4 * rr + 2] * scale, dqacc[i][4 * rr + 3] * scale)});
      }
    OStage::store(ost, rdq, (uint32_t)q0, row_bytes, 0, lane);
  }
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_t(const BwdParams& p, hipStream_t s) {
  const long nrows = p.cu ? (long)p.T * p.H : (long)p.B * p.N * p.H;
  const int rpb = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<BF16, D>), dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nkvt = (p.N + kWaves * 32 - 1) / (kWaves * 32);
  hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, CAUSAL>), dim3((unsigned)(p.B * p.Hkv * nkvt)), dim3(256), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  constexpr int qw = DqCfg<D>::WAVES;
  const int nqt = (p.N + qw * 32 - 1) / (qw * 32);
  hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, CAUSAL>), dim3((unsigned)(p.B * p.H * nqt)), dim3(64 * qw), 0, s, p);
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
