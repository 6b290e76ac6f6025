// Forward exact attention for gfx950: one workgroup per (query tile, head, batch).
//
// Method (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention"): the query tile
// Q_i stays resident while K_j, V_j tiles stream past it (Symbol Map); each tile gives
// S = Q_i K_j^T, the online softmax keeps a running row maximum m_i and sum l_i, P~ V_j is
// added to the output numerator, and the epilogue divides by l_i and stores O_i and
// L_i = m_i + log(l_i) ("Putting It Together", steps 2-7).
//
// gfx950 design (the Hopper producer/consumer, TMA and WGMMA machinery is prior art only):
//  * d = 64, 128: 8 waves x 32 query rows = 256 rows per workgroup, one workgroup per CU
//    (two waves per SIMD), sharing a three-stage K ring and a four-stage V ring; key tiles
//    of BC = 64. Ping-pong between the two waves of a SIMD (same page, Deep Dive, "Ping-pong
//    scheduling"): the second wave takes each tile's barrier between its
//    score block and its P~V block, so on every SIMD one wave's exponentials run beside
//    the other wave's P~V MFMAs; the extra V stage covers the late reads. d = 256 needs
//    more than 256 registers: 4 waves (one per SIMD) and two-stage rings.
//  * K and V tiles go from HBM straight into the LDS ring by DMA (buffer_load_dwordx4 ...
//    lds) with no register staging; with NS stages each tile is requested NS-2 loop
//    iterations before the one whose end must see it landed, so the DMA latency hides under
//    several tiles of work. One barrier per tile separates the stages. Rows past N arrive
//    as zeros (buffer range check).
//  * Scores are produced transposed, S^T = K Q^T (MFMA 32x32x16): each lane then owns ONE
//    query row (column l%32 of the accumulator) and 16 keys of each 32-key block, so the
//    row maximum is an in-lane reduction plus one permlane32 swap, and the row sum stays a
//    per-lane partial until the epilogue.
//  * The score accumulator is the B operand of O^T += V^T P^T without any lane exchange:
//    accumulator r of lane half hf is key 8*(r/4) + 4*hf + r%4, and the V^T operand is
//    gathered from the row-major V tile by two LDS transpose reads (ds_read_b64_tr_b16)
//    pointed at exactly those keys.
//  * Online softmax in the exp2 domain (scores scaled by scale*log2 e with one FMA), and
//    a lazy rescale: the reference maximum only moves (and O, l are only rescaled) when a
//    row's maximum grows by more than 2^8, decided per wave with a ballot. Any reference
//    value gives the same exact O and L; this one keeps P~ <= 256 and skips most rescales.
//  * Only tiles that touch the causal diagonal or the ragged end run the masking code.
//  * Causal: tiles past the diagonal are never loaded; longest query tiles launch first;
//    waves whose rows all precede a tile skip its math.
//  * Block ids are remapped so that all query tiles of a head run on one XCD (shared L2).
#include <type_traits>

#include "attn_launch.h"
#include "attn_lds.h"

namespace attn {

namespace {

template <int D, bool SMALL = false> struct FwdCfg;
// BC: keys per tile; WAVES: waves per workgroup; STAGES: depth of the K ring (the V ring has
// one more stage under ping-pong); PP: ping-pong schedule between the two waves of each
// SIMD (needs two waves per SIMD); WGS: workgroups per CU.
// The default form is one workgroup per CU (two waves per SIMD at d <= 128). SMALL is for
// grids too short to keep one such workgroup per CU busy (short sequences, few heads): half
// the query rows per workgroup and two workgroups per CU, so that one workgroup's start-up
// loads and epilogue overlap the other's tiles and twice as many CUs get work.
template <> struct FwdCfg<64> { static constexpr int BC = 64, WAVES = 8, STAGES = 3, WGS = 1; static constexpr bool PP = true; };
template <> struct FwdCfg<128> { static constexpr int BC = 64, WAVES = 8, STAGES = 3, WGS = 1; static constexpr bool PP = true; };
template <> struct FwdCfg<256> { static constexpr int BC = 64, WAVES = 4, STAGES = 2, WGS = 1; static constexpr bool PP = false; };
template <> struct FwdCfg<64, true> { static constexpr int BC = 64, WAVES = 4, STAGES = 2, WGS = 2; static constexpr bool PP = false; };
template <> struct FwdCfg<128, true> { static constexpr int BC = 64, WAVES = 4, STAGES = 2, WGS = 2; static constexpr bool PP = false; };

constexpr int kQW = 32;                  // query rows per wave
template <int D, bool SMALL = false> constexpr int fwd_rows() { return FwdCfg<D, SMALL>::WAVES * kQW; }   // per workgroup
template <int D, bool SMALL> constexpr int fwd_threads() { return 64 * FwdCfg<D, SMALL>::WAVES; }
template <int D, bool SMALL> constexpr int fwd_wgs() { return FwdCfg<D, SMALL>::WGS; }
constexpr float kTau = 8.0f;             // lazy-rescale threshold (log2 units)
constexpr float kLn2 = 0.69314718055994530942f;

// Scores of one key tile for this wave: s[kb] = K[kb*32 .. +31] Q^T (32 keys x 32 queries).
template <bool BF16, int D, int NKB>
__device__ __forceinline__ void tile_scores(f32x16 (&s)[NKB], const char* kl, const u32x4 (&qreg)[D / 16]) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) s[kb] = mfma32x16<BF16>(lds_k<D>(kl, kb, kk), qreg[kk], s[kb]);
  }
}

// Causal / ragged mask of a tile: keys past N or past the query become -inf.
template <bool CAUSAL, int NKB>
__device__ __forceinline__ void tile_mask(f32x16 (&s)[NKB], int k0, int N, int qrow, int hf) {
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
    }
}

// Row maximum (in the exp2 domain) of a tile; -inf if every key of the row is masked.
template <int NKB>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[NKB], float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = xhalf_max(mx);
  return mx == -INFINITY ? -INFINITY : mx * c;
}

// P~ = exp2(s*c - m) packed to 16-bit MFMA B operands (16 keys per operand); returns the
// lane's partial row sum of the fp32 P~.
template <bool BF16, bool EDGE, int NKB>
__device__ __forceinline__ float tile_exp(const f32x16 (&s)[NKB], u32x4 (&pk)[2 * NKB], float c, float m_use) {
  float psum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      float e[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float x = s[kb][8 * h2 + t];
        e[t] = fast_exp2(fmaf(x, c, -m_use));
        if constexpr (EDGE) e[t] = (x == -INFINITY) ? 0.f : e[t];
        psum += e[t];
      }
      pk[2 * kb + h2] = u32x4{pack2<BF16>(e[0], e[1]), pack2<BF16>(e[2], e[3]), pack2<BF16>(e[4], e[5]),
                              pack2<BF16>(e[6], e[7])};
    }
  return psum;
}

// O^T += V^T P^T for one tile (V row-major in LDS, gathered by transpose reads). `vl` is
// restrict: the compiler can then tell that these reads do not touch the stages the DMA in
// flight is filling; otherwise it waits for every outstanding DMA (vmcnt(0)) before the
// first transpose read, which drains the ring's prefetch every tile.
template <bool BF16, int D, int NKB>
__device__ __forceinline__ void tile_pv(f32x16 (&oacc)[D / 32], const char* __restrict__ vl, const u32x4 (&pk)[2 * NKB]) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int cidx = 0; cidx < 2 * NKB; ++cidx) oacc[i] = mfma32x16<BF16>(lds_vt<D>(vl, cidx, i), pk[cidx], oacc[i]);
}

// SPLIT: the workgroup covers part `split` (tiles split*T .. split*T + T - 1, T =
// p.split_tiles) of its query tile's key tiles; slots past the tile's last part exit at
// once. With two or more parts it writes the part's O/l and L (natural log) to p.o_part,
// p.lse_part (rows with no key in the part: L = -inf); a tile with one part writes O, L.
template <bool BF16, int D, bool CAUSAL, bool SPLIT = false, bool SMALL = false>
__global__ __launch_bounds__((fwd_threads<D, SMALL>()), (fwd_wgs<D, SMALL>())) void fwd_kernel(FwdParams p) {
  using Cfg = FwdCfg<D, SMALL>;
  constexpr int BC = Cfg::BC;
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int kWaves = Cfg::WAVES;
  constexpr int NS = Cfg::STAGES;
  constexpr int kBR = fwd_rows<D, SMALL>();
  using KPlan = DmaPlan<D, BC, k_pitch<D>(), kWaves>;
  using VPlan = DmaPlan<D, BC, v_pitch<D>(), kWaves>;
  // DMA instructions every wave issues per K / V tile (some issue one more)
  constexpr int KMIN = KPlan::NI / kWaves, VMIN = VPlan::NI / kWaves;
  static_assert(KMIN >= 1 && VMIN >= 1, "every wave takes part in each tile's DMA");

  // Ping-pong: the second wave of each SIMD runs the P~V half of every fast tile one
  // barrier interval late, so that on each SIMD one wave exponentiates while the other
  // multiplies.
  constexpr bool PP = Cfg::PP;
  constexpr int VS = NS + (PP ? 1 : 0);
  // K ring (NS stages) then V ring (VS stages); tile t lives in stage t % NS (t % VS).
  // Loop iteration j reads K(j+1) and V(j) (and V(j-1) in the late waves), and requests
  // V(j+NS-1) and K(j+NS) into stages no wave reads after the previous barrier.
  constexpr int KBYTES = KPlan::BYTES, VBYTES = VPlan::BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[NS * KBYTES + VS * VBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keeps loop control scalar
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H;
  const int nqt = (p.N + kBR - 1) / kBR;   // p.N: the (longest) sequence length

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int split = SPLIT ? work % p.splits : 0;   // parts of one query tile are neighbours
  const int qwork = SPLIT ? work / p.splits : work;
  const int qi = qwork % nqt;
  const int bh = spread_pair(qwork / nqt, p.B * H, !SPLIT && p.cu != nullptr);
  const int h = bh % H, b = bh / H;
  const SeqView sv = seq_view(p.cu, b, p.N, p.T);
  const int N = sv.len;
  const int qt = CAUSAL ? nqt - 1 - qi : qi;
  if (qt * kBR >= N) return;   // a shorter sequence of a variable-length batch: nothing here
  const int q0 = qt * kBR + wave * kQW;
  const int qrow = q0 + l32;

  // Per-(batch, head) buffer views: offset = row * row_bytes + byte within the head's row.
  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const size_t head_off = ((size_t)sv.start * H + h) * D * 2;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D * 2;
  const auto rq = make_rsrc((const char*)p.q + head_off, nrec);
  const auto ro = make_rsrc((const char*)p.o + head_off, nrec);
  // K and V: [B][N][Hkv][D], head h / (H / Hkv) (grouped key/value heads; Hkv = H is plain)
  const int Hkv = p.Hkv, kvh = h / (H / Hkv);
  const uint32_t kv_row_bytes = (uint32_t)Hkv * D * 2;
  const size_t kv_head_off = ((size_t)sv.start * Hkv + kvh) * D * 2;
  const uint32_t kv_nrec = (uint32_t)N * kv_row_bytes - (uint32_t)kvh * D * 2;

  const int kend = CAUSAL ? min(N, (qt + 1) * kBR) : N;
  const int nkt_all = (kend + BC - 1) / BC;
  // key tiles t0 .. t0 + nkt - 1 (global indices) of this workgroup: all, or one part
  int t0 = 0, nkt = nkt_all, parts = 1;
  if constexpr (SPLIT) {
    parts = (nkt_all + p.split_tiles - 1) / p.split_tiles;
    if (split >= parts) return;   // an unused slot (uniform over the workgroup, before any barrier)
    t0 = split * p.split_tiles;
    nkt = min(nkt_all, t0 + p.split_tiles) - t0;
  }
  // tiles this wave computes: causal rows stop at the diagonal tile; rows past N compute
  // none. Every tile a wave computes holds an unmasked key of each of its rows (a tile
  // starts at or before the wave's first row), so no computed row is fully masked.
  const int nkt_w_all = q0 >= N ? 0 : CAUSAL ? min(nkt_all, (q0 + kQW - 1) / BC + 1) : nkt_all;
  const int nkt_w = max(0, min(nkt, nkt_w_all - t0));
  // Stage offsets pass through readfirstlane: opaque to loop strength reduction, which would
  // otherwise keep one induction register per operand address.
  auto kst = [&](int j) { return smem + __builtin_amdgcn_readfirstlane((j % NS) * KBYTES); };
  auto vst = [&](int j) { return smem + NS * KBYTES + __builtin_amdgcn_readfirstlane((j % VS) * VBYTES); };
  const int k_lane = k_lane_off<D>(lane), v_lane = v_lane_off<D>(lane);
  auto is_edge = [&](int j) { const int k0 = (t0 + j) * BC; return (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0); };
  uint32_t kvoff[KPlan::NPW], vvoff[VPlan::NPW];
  dma_init<KPlan, kWaves>(kvoff, kv_row_bytes, wave, lane);
  dma_init<VPlan, kWaves>(vvoff, kv_row_bytes, wave, lane);
  const char* kbase = (const char*)p.k + kv_head_off;
  const char* vbase = (const char*)p.v + kv_head_off;
  auto dma_k = [&](int t) { dma_issue<KPlan, kWaves>(kvoff, kst(t), kbase, (t0 + t) * BC, kv_row_bytes, kv_nrec, wave); };
  auto dma_v = [&](int t) { dma_issue<VPlan, kWaves>(vvoff, vst(t), vbase, (t0 + t) * BC, kv_row_bytes, kv_nrec, wave); };

  // Q^T operand: lane holds query q0 + l32, dims 16*ks + 8*hf .. +7.
  u32x4 qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qreg[ks] = buf_load16(rq, (uint32_t)qrow * row_bytes + (16 * ks + 8 * hf) * 2);

  // Prologue requests K(0), then the pairs V(t), K(t+1) for t = 0 .. NS-2; loop iteration
  // j requests the pair V(j+NS-1), K(j+NS). Before iteration j (and before the loop, j = 0)
  // K(j+1) and V(j) must have landed: everything but the pairs requested for t >= j+1 may
  // stay in flight. This wave's share of a tile's DMA instructions: blocks wave, wave + W,
  // ... below NI.
  const int nk_w = KMIN + (wave < KPlan::NI % kWaves ? 1 : 0);
  const int nv_w = VMIN + (wave < VPlan::NI % kWaves ? 1 : 0);
  constexpr int KEEP_MAX = (NS - 2) * (KMIN + VMIN + 2);
  auto wait_before = [&](int j) {   // wait until K(j+1) and V(j) are in LDS (this wave's part)
    int keep = 0;
#pragma unroll
    for (int t = 1; t <= NS - 2; ++t) keep += (j + t < nkt ? nv_w : 0) + (j + t + 1 < nkt ? nk_w : 0);
    // Away from the end of the key range every tile of the batch exists: keep the count
    // of the waves with the fewest DMA instructions, a constant. The other waves then also
    // wait for the first one or two of their batch, issued at the start of the tile
    // (waiting longer is always safe); a count chosen at run time would cost a chain of
    // compares and branches per tile.
    if (j + NS - 1 < nkt) wait_dma_keep<(NS - 2) * (KMIN + VMIN)>();
    else wait_dma_keep_rt<KEEP_MAX>(keep);
  };
  if (nkt > 0) dma_k(0);   // a split-KV part can be empty: then no tile is loaded at all

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.c;

#pragma unroll
  for (int t = 0; t <= NS - 2; ++t) {
    if (t < nkt) dma_v(t);
    if (t + 1 < nkt) dma_k(t + 1);
  }
  // Q is waited for only now: its load and the first tiles' DMA share one HBM round trip
  // (4-6% on 512-token sequences, where a workgroup has only 8 key tiles to amortise it).
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) settle(qreg[ks]);
  wait_before(0);
  __syncthreads();

  // Two-stage software pipeline (per wave): while the scores of tile j+1 are being
  // multiplied out on the MFMA pipe, the VALU exponentiates tile j; while P~(j) V(j) runs,
  // the VALU takes the row maximum of tile j+1.
  f32x16 sc[NKB], sn[NKB];
  float mx_next = -INFINITY;
  if (nkt_w > 0) {
    tile_scores<BF16, D, NKB>(sc, kst(0) + k_lane, qreg);
    if (is_edge(0)) tile_mask<CAUSAL, NKB>(sc, t0 * BC, N, qrow, hf);
    mx_next = tile_max<NKB>(sc, c);
  }
  // the first prefetch overwrites the stage of K(0), which the prologue just read
  ring_barrier();

  auto prefetch = [&](int j) {
    if (j + NS - 1 < nkt) dma_v(j + NS - 1);
    if (j + NS < nkt) dma_k(j + NS);
  };
  // End of iteration j: iteration j+1 reads K(j+2) and V(j+1).
  auto end_tile = [&](int j) {
    wait_before(j + 1);
    ring_barrier();
  };
  // the maximum of tile j (taken one step earlier) may move the reference: rescale O and l
  auto rescale = [&]() {
    const float m_cand = fmaxf(m_run, mx_next);
    if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kTau)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_cand);
      m_run = m_cand;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    }
  };

  // Interior tiles (neither tile j nor j+1 masked): the pipelined form, with the instruction
  // order written out. Block 1 issues one S(j+1) MFMA per step and, under it, exponentiates EPS scores of
  // tile j (packing the first 16-key chunk of P~ as soon as it is complete). Block 2 issues
  // one P~(j)V(j) MFMA per step and, under it, packs the next chunk of P~ (one conversion
  // per step, ahead of the step that consumes it), adds the row-sum terms and folds tile
  // j+1 into the row maximum. This splits the VALU work about evenly between the blocks.
  // LDS operands are fetched PF steps ahead; sched_barrier fences keep each step's order.
  constexpr int S1 = NKB * NKS;       // MFMAs in block 1
  constexpr int S2 = NDB * 2 * NKB;   // MFMAs in block 2
  constexpr int EPS = 16 * NKB / S1;  // scores exponentiated per block-1 step (256/d)
  constexpr int MPS = 16 * NKB / S2;  // scores summed and folded into the max per block-2 step (512/d)
  constexpr int PF = 2;
  constexpr int C0 = 8 / EPS;         // block-1 step that packs the first conversion of chunk 0
  static_assert(EPS * S1 == 16 * NKB && MPS * S2 == 16 * NKB && EPS >= 1 && (MPS == 1 || MPS % 2 == 0), "step split");
  static_assert(C0 + 4 <= S1 && NDB % 2 == 0 && NDB <= 8, "chunk 0 packs inside block 1");
  // P~ of the tile in flight: fp32 values, then 16-bit pairs (word 4q + u of 16-key chunk q
  // holds keys 8q + 2u, 8q + 2u + 1). Scalars, not vectors: a vector filled one element at a
  // time would keep its previous value alive around the loop.
  float e[16 * NKB];
  uint32_t pw[8 * NKB];
  auto pack = [&](int q, int u) { pw[4 * q + u] = pack2<BF16>(e[8 * q + 2 * u], e[8 * q + 2 * u + 1]); };
  // Block 1 of tile jj: S(jj+1) = K(jj+1) Q^T into nxt, P~(jj) = exp2(cur*c - m) into e.
  auto blk1 = [&](int jj, const f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB]) __attribute__((always_inline)) {
    const float m_use = m_run;
    const char* kn = kst(jj + 1) + k_lane;
    u32x4 kop[S1];
    __builtin_amdgcn_sched_barrier(0);
    // step t multiplies key block t % NKB at k-step t / NKB: consecutive MFMAs accumulate
    // into different registers.
#pragma unroll
    for (int t = 0; t < PF; ++t) kop[t] = lds_k<D>(kn, t % NKB, t / NKB);
#pragma unroll
    for (int t = 0; t < S1; ++t) {
      if (t + PF < S1) kop[t + PF] = lds_k<D>(kn, (t + PF) % NKB, (t + PF) / NKB);
      const int kb = t % NKB, kk = t / NKB;
      nxt[kb] = mfma32x16<BF16>(kop[t], qreg[kk], kk == 0 ? f32x16{} : nxt[kb]);
#pragma unroll
      for (int u = 0; u < EPS; ++u) {
        const int i = EPS * t + u;
        e[i] = fast_exp2(fmaf(cur[i >> 4][i & 15], c, -m_use));
        pin(e[i]);   // computed here: the compiler would sink it to its use in block 2
      }
      if (t >= C0 && t < C0 + 4) {
        pack(0, t - C0);
        pin(pw[t - C0]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Block 2 of tile jj: O^T += V(jj)^T P~(jj)^T, the row sum of P~(jj), and the row maximum
  // of the scores nxt = S(jj+1) that block 1 of tile jj produced. `vc` (V(jj) in LDS, this
  // lane's base) is restrict for the reason given at tile_pv.
  auto blk2 = [&](const char* __restrict__ vc, const f32x16 (&nxt)[NKB]) __attribute__((always_inline)) {
    u32x4 vop[S2];
    float mx = -INFINITY, psum = 0.f;
    __builtin_amdgcn_sched_barrier(0);
    // step t adds key chunk t / NDB into output block t % NDB (different accumulators in turn)
#pragma unroll
    for (int t = 0; t < PF; ++t) vop[t] = lds_vt<D>(vc, t / NDB, t % NDB);
#pragma unroll
    for (int t = 0; t < S2; ++t) {
      if (t + PF < S2) vop[t + PF] = lds_vt<D>(vc, (t + PF) / NDB, (t + PF) % NDB);
      const int i = t % NDB, cidx = t / NDB;
      oacc[i] = mfma32x16<BF16>(vop[t], u32x4{pw[4 * cidx], pw[4 * cidx + 1], pw[4 * cidx + 2], pw[4 * cidx + 3]}, oacc[i]);
      // chunk cidx + 1 is consumed from step NDB * (cidx + 1): convert it during chunk cidx,
      // CPS conversions every SS-th step
      constexpr int CPS = NDB >= 4 ? 1 : 4 / NDB, SS = NDB >= 4 ? NDB / 4 : 1;
      if (cidx + 1 < 2 * NKB && (t % NDB) % SS == 0) {
#pragma unroll
        for (int v = 0; v < CPS; ++v) pack(cidx + 1, ((t % NDB) / SS) * CPS + v);
      }
      if constexpr (MPS == 1) {
        psum += e[t];
        mx = fmaxf(mx, nxt[t >> 4][t & 15]);
      } else {
#pragma unroll
        for (int u = 0; u < MPS; u += 2) {
          const int i2 = MPS * t + u;
          psum += e[i2];
          psum += e[i2 + 1];
          mx = max3(mx, nxt[i2 >> 4][i2 & 15], nxt[(i2 + 1) >> 4][(i2 + 1) & 15]);
        }
      }
      pin(psum);   // keep the sum's adds in this step (the compiler would sink them)
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += psum;
    mx = xhalf_max(mx);
    mx_next = mx * c;
  };
  // Tile jj runs the fast path when tiles jj and jj+1 need no mask: jj + 1 < nkt_w and
  // !is_edge(jj + 1) (masking only ever starts near the end of a wave's key range, so the
  // fast tiles are a prefix). The tests are written out in the loop: a helper lambda for
  // them changes how the loops are optimised and costs registers in the causal kernels.
  // One fast iteration. The late waves (ping-pong) take the barrier that ends iteration jj
  // between the two blocks: their block 2 of tile jj then runs after that barrier, beside
  // the early waves' block 1 of tile jj+1, so on each SIMD one wave's exponentials overlap
  // the other wave's P~V MFMAs. The barrier count is unchanged; V(jj) is read one barrier
  // interval later, which the extra V stage covers.
  auto fast_iter = [&](auto late, int jj, f32x16 (&cur)[NKB], f32x16 (&nxt)[NKB]) __attribute__((always_inline)) {
    prefetch(jj);
    rescale();
    blk1(jj, cur, nxt);
    if constexpr (decltype(late)::value) end_tile(jj);
    blk2(vst(jj) + v_lane, nxt);
    if constexpr (!decltype(late)::value) end_tile(jj);
  };
  int j = 0;
  auto fast_loop = [&](auto late) __attribute__((always_inline)) {
    for (; j + 2 < nkt_w && !is_edge(j + 2); j += 2) {   // sc/sn swap roles: no copies
      fast_iter(late, j, sc, sn);
      fast_iter(late, j + 1, sn, sc);
    }
    if (j + 1 < nkt_w && !is_edge(j + 1)) {
      fast_iter(late, j, sc, sn);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sc[kb] = sn[kb];
      ++j;
    }
  };
  // Waves w and w + W/2 share a SIMD (waves are placed on the SIMDs round-robin).
  if (PP && wave >= kWaves / 2) fast_loop(std::true_type{});
  else fast_loop(std::false_type{});
  // Remaining tiles, in order: masked tiles and the tail of the key range (and, for waves
  // with nothing left to compute, only the ring bookkeeping every wave takes part in).
  for (; j < nkt; ++j) {
    prefetch(j);
    if (j < nkt_w) {
      rescale();
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      u32x4 pk[2 * NKB];
      if (is_edge(j)) l_run += tile_exp<BF16, true, NKB>(sc, pk, c, m_use);
      else l_run += tile_exp<BF16, false, NKB>(sc, pk, c, m_use);
      tile_pv<BF16, D, NKB>(oacc, vst(j) + v_lane, pk);
      if (j + 1 < nkt_w) {
        tile_scores<BF16, D, NKB>(sc, kst(j + 1) + k_lane, qreg);
        if (is_edge(j + 1)) tile_mask<CAUSAL, NKB>(sc, (t0 + j + 1) * BC, N, qrow, hf);
        mx_next = tile_max<NKB>(sc, c);
      }
    }
    end_tile(j);
  }

  if (SPLIT && parts > 1) {
    const size_t part = ((size_t)split * p.B + b) * H + h;   // [S][B][H]
    if (qrow < N) {
      if (nkt_w > 0) {
        const float l_tot = xhalf_sum(l_run);
        const float inv = 1.0f / l_tot;
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float* orow = p.o_part + (part * N + qrow) * D;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
            *(f32x4*)(orow + i * 32 + 8 * rr + 4 * hf) =
                f32x4{oacc[i][4 * rr] * inv, oacc[i][4 * rr + 1] * inv, oacc[i][4 * rr + 2] * inv, oacc[i][4 * rr + 3] * inv};
        if (hf == 0) p.lse_part[part * N + qrow] = (m_use + fast_log2(l_tot)) * kLn2;
      } else if (hf == 0) {
        p.lse_part[part * N + qrow] = -INFINITY;
      }
    }
    return;
  }
  // O leaves through the ring's LDS, each wave in its own area: the last end_tile() waited for
  // every DMA and passed a barrier after every wave's last operand read.
  using OStage = RowStage<2 * D>;
  static_assert(kQW == 32 && kWaves * OStage::BYTES <= (int)sizeof(smem), "O staging fits the ring");
  if (nkt_w > 0) {
    const float l_tot = xhalf_sum(l_run);
    const float inv = 1.0f / l_tot;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    char* ost = smem + wave * OStage::BYTES;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        u32x2 v = {pack2<BF16>(oacc[i][4 * rr + 0] * inv, oacc[i][4 * rr + 1] * inv),
                   pack2<BF16>(oacc[i][4 * rr + 2] * inv, oacc[i][4 * rr + 3] * inv)};
        OStage::put(ost, l32, d0 * 2, v);
      }
    OStage::store(ost, ro, (uint32_t)q0, row_bytes, 0, lane);
    if (hf == 0 && qrow < N) p.lse[stat_row(p.cu, p.T, b, H, h, sv) + qrow] = (m_use + fast_log2(l_tot)) * kLn2;
  }
}

// Merge of the split-KV parts, one row per D/8 threads (8 dims each): L = log sum_s e^{L_s},
// O = sum_s e^{L_s - L} O_s over the parts of the row's query tile, parts with L_s = -inf
// skipped (their O_s is never read). Rows of single-part tiles were written directly.
constexpr int kMaxSplits = 16;
template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPB = 256 / TPR;
  const int H = p.H, N = p.N;
  const size_t rows = (size_t)p.B * H * N;
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / TPR;   // (b, h, n) order
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  const int n = (int)(row % N);
  const int qt = n / fwd_rows<D>();
  const int kend = CAUSAL ? min(N, (qt + 1) * fwd_rows<D>()) : N;
  const int nkt_all = (kend + FwdCfg<D>::BC - 1) / FwdCfg<D>::BC;
  const int S = (nkt_all + p.split_tiles - 1) / p.split_tiles;
  if (S <= 1) return;
  const size_t bh = row / N;
  const int h = (int)(bh % H), b = (int)(bh / H);
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, p.lse_part[(size_t)s * rows + row]);
  float sum = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float ls = p.lse_part[(size_t)s * rows + row];
    if (ls == -INFINITY) continue;
    const float w = __expf(ls - m);
    sum += w;
    const f32x4* src = (const f32x4*)(p.o_part + ((size_t)s * rows + row) * D + 8 * c);
    const f32x4 lo = src[0], hi = src[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += w * lo[e];
      acc[4 + e] += w * hi[e];
    }
  }
  const float inv = 1.0f / sum;
  const u32x4 out = {pack2<BF16>(acc[0] * inv, acc[1] * inv), pack2<BF16>(acc[2] * inv, acc[3] * inv),
                     pack2<BF16>(acc[4] * inv, acc[5] * inv), pack2<BF16>(acc[6] * inv, acc[7] * inv)};
  *(u32x4*)((char*)p.o + ((((size_t)b * N + n) * H + h) * D + 8 * c) * 2) = out;
  if (c == 0) p.lse[row] = m + __logf(sum);
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_split(const FwdParams& p, hipStream_t s) {
  static_assert(FwdCfg<D>::BC == 64, "split_tiles is computed for 64-key tiles");
  const int nqt = (p.N + fwd_rows<D>() - 1) / fwd_rows<D>();
  const dim3 grid((unsigned)(p.B * p.H * nqt * p.splits));
  hipLaunchKernelGGL((fwd_kernel<BF16, D, CAUSAL, true>), grid, dim3(64 * FwdCfg<D>::WAVES), 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int RPB = 256 / (D / 8);
  const size_t rows = (size_t)p.B * p.H * p.N;
  hipLaunchKernelGGL((fwd_merge_kernel<BF16, D, CAUSAL>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <bool BF16, int D, bool CAUSAL, bool SMALL>
hipError_t launch_g(const FwdParams& p, hipStream_t s) {
  const int nqt = (p.N + fwd_rows<D, SMALL>() - 1) / fwd_rows<D, SMALL>();
  const dim3 grid((unsigned)(p.B * p.H * nqt));
  hipLaunchKernelGGL((fwd_kernel<BF16, D, CAUSAL, false, SMALL>), grid, dim3(64 * FwdCfg<D, SMALL>::WAVES), 0, s, p);
  return hipGetLastError();
}

// The small form when sequences are short (a workgroup's start-up is a large share of its
// work) or the default grid would leave CUs idle (fewer workgroups than the 256 CUs), and
// always at d = 64, where the exponentials bound the kernel and two independent workgroups
// per CU keep the VALU busier than the ping-pong pair of one workgroup (6-8% faster at
// N = 2048 and 8192, measured).
template <bool BF16, int D, bool CAUSAL>
hipError_t launch_t(const FwdParams& p, hipStream_t s) {
  if constexpr (D <= 128) {
    const long nwg = (long)p.B * p.H * ((p.N + fwd_rows<D>() - 1) / fwd_rows<D>());
    if (D == 64 || p.N <= 1024 || nwg < 256) return launch_g<BF16, D, CAUSAL, true>(p, s);
  }
  return launch_g<BF16, D, CAUSAL, false>(p, s);
}

template <bool BF16, int D>
hipError_t launch_c(bool causal, const FwdParams& p, hipStream_t s) {
  return causal ? launch_t<BF16, D, true>(p, s) : launch_t<BF16, D, false>(p, s);
}

template <bool BF16>
hipError_t launch_d(int d, bool causal, const FwdParams& p, hipStream_t s) {
  switch (d) {
    case 64: return launch_c<BF16, 64>(causal, p, s);
    case 128: return launch_c<BF16, 128>(causal, p, s);
    case 256: return launch_c<BF16, 256>(causal, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd(bool bf16, int d, bool causal, const FwdParams& p, hipStream_t s) {
  return bf16 ? launch_d<true>(d, causal, p, s) : launch_d<false>(d, causal, p, s);
}

template <bool BF16>
hipError_t launch_split_d(int d, bool causal, const FwdParams& p, hipStream_t s) {
  switch (d) {
    case 64: return causal ? launch_split<BF16, 64, true>(p, s) : launch_split<BF16, 64, false>(p, s);
    case 128: return causal ? launch_split<BF16, 128, true>(p, s) : launch_split<BF16, 128, false>(p, s);
    case 256: return causal ? launch_split<BF16, 256, true>(p, s) : launch_split<BF16, 256, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_splitkv(bool bf16, int d, bool causal, const FwdParams& p, hipStream_t s) {
  if (p.splits < 1 || p.splits > kMaxSplits) return hipErrorInvalidValue;
  FwdParams q = p;
  const int nkt_max = (p.N + 63) / 64;   // key tiles of the longest query tile (BC = 64)
  q.split_tiles = (nkt_max + p.splits - 1) / p.splits;
  return bf16 ? launch_split_d<true>(d, causal, q, s) : launch_split_d<false>(d, causal, q, s);
}

}  // namespace attn
