// Forward exact attention for gfx950: one workgroup per (query tile, head, batch).
//
// Method (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention"): the query tile
// Q_i stays resident while K_j, V_j tiles stream past it (Symbol Map); each tile gives
// S = Q_i K_j^T, the online softmax keeps a running row maximum m_i and sum l_i, P~ V_j is
// added to the output numerator, and the epilogue divides by l_i and stores O_i and
// L_i = m_i + log(l_i) ("Putting It Together", steps 2-7).
//
// gfx950 design (the Hopper producer/consumer, TMA and WGMMA machinery is prior art only):
//  * 4 waves x 32 query rows = 128 rows per workgroup, two workgroups per CU (two waves per
//    SIMD, so one wave's softmax runs while the other's MFMAs do); key tiles of BC = 64
//    (d = 64: 128). d = 256 needs more than 256 registers and runs one wave per SIMD.
//  * K and V tiles go from HBM straight into a two-stage LDS ring by DMA
//    (buffer_load_dwordx4 ... lds), one tile ahead, with no register staging; one barrier
//    per tile separates the stages. Rows past N arrive as zeros (buffer range check).
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

template <int D> struct FwdCfg;
// BC: keys per tile; OCC: waves per SIMD the register budget is sized for.
template <> struct FwdCfg<64> { static constexpr int BC = 128, OCC = 2; };
template <> struct FwdCfg<128> { static constexpr int BC = 64, OCC = 2; };
template <> struct FwdCfg<256> { static constexpr int BC = 64, OCC = 1; };

constexpr int kWaves = 4;
constexpr int kQW = 32;                  // query rows per wave
constexpr int kBR = kWaves * kQW;        // query rows per workgroup
constexpr float kTau = 8.0f;             // lazy-rescale threshold (log2 units)
constexpr float kLn2 = 0.69314718055994530942f;

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256, FwdCfg<D>::OCC) void fwd_kernel(FwdParams p) {
  constexpr int BC = FwdCfg<D>::BC;
  constexpr int TB = BC * 2 * D;         // bytes of one K or V tile
  constexpr int STAGE = 2 * TB;
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int H = p.H, N = p.N;
  const int nqt = (N + kBR - 1) / kBR;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qi = work % nqt;
  const int bh = work / nqt;
  const int h = bh % H, b = bh / H;
  const int qt = CAUSAL ? nqt - 1 - qi : qi;
  const int q0 = qt * kBR + wave * kQW;

  // Per-(batch, head) buffer views: offset = row * row_bytes + byte within the head's row.
  const uint32_t row_bytes = (uint32_t)H * D * 2;
  const size_t head_off = ((size_t)b * N * H + h) * D * 2;
  const uint32_t nrec = (uint32_t)N * row_bytes - (uint32_t)h * D * 2;
  const auto rq = make_rsrc((const char*)p.q + head_off, nrec);
  const auto rk = make_rsrc((const char*)p.k + head_off, nrec);
  const auto rv = make_rsrc((const char*)p.v + head_off, nrec);
  const auto ro = make_rsrc((const char*)p.o + head_off, nrec);

  const int kend = CAUSAL ? min(N, (qt + 1) * kBR) : N;
  const int nkt = (kend + BC - 1) / BC;
  auto fetch = [&](int k0, int stage) {
    char* st = smem + stage * STAGE;
    dma_tile<D, BC, false, kWaves>(st, rk, k0, row_bytes, wave, lane);
    dma_tile<D, BC, true, kWaves>(st + TB, rv, k0, row_bytes, wave, lane);
  };
  fetch(0, 0);

  // Q^T operand: lane holds query q0 + l32, dims 16*ks + 8*hf .. +7.
  u32x4 qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qreg[ks] = buf_load16(rq, (uint32_t)(q0 + l32) * row_bytes + (16 * ks + 8 * hf) * 2);

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const bool wave_live = q0 < N;
  const int qrow = q0 + l32;
  const float c = p.c;

  wait_dma();
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int k0 = j * BC;
    if (j + 1 < nkt) fetch(k0 + BC, (j + 1) & 1);
    const char* ks = smem + (j & 1) * STAGE;
    const char* vs = ks + TB;
    const bool skip = !wave_live || (CAUSAL && k0 > q0 + kQW - 1);
    auto tile = [&](auto edge_tag) {
      constexpr bool EDGE = decltype(edge_tag)::value;
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) s[kb] = mfma32x16<BF16>(lds_row<D>(ks, kb * 32 + l32, kk, hf), qreg[kk], s[kb]);
      }
      if constexpr (EDGE) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = xhalf_max(mx);
      float mt = mx * c;
      if constexpr (EDGE) mt = (mx == -INFINITY) ? -INFINITY : mt;
      const float m_cand = fmaxf(m_run, mt);
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kTau)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_cand);
        m_run = m_cand;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float e = fast_exp2(fmaf(s[kb][r], c, -m_use));
          if constexpr (EDGE) e = (s[kb][r] == -INFINITY) ? 0.f : e;
          s[kb][r] = e;
          psum += e;
        }
      l_run += psum;
      u32x4 pk[BC / 16];
#pragma unroll
      for (int cidx = 0; cidx < BC / 16; ++cidx) {
        const int kb = cidx >> 1, base = (cidx & 1) * 8;
        pk[cidx] = u32x4{pack2<BF16>(s[kb][base + 0], s[kb][base + 1]), pack2<BF16>(s[kb][base + 2], s[kb][base + 3]),
                         pack2<BF16>(s[kb][base + 4], s[kb][base + 5]), pack2<BF16>(s[kb][base + 6], s[kb][base + 7])};
      }
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int cidx = 0; cidx < BC / 16; ++cidx)
          oacc[i] = mfma32x16<BF16>(lds_tr<D>(vs, 16 * cidx, 32 * i, lane), pk[cidx], oacc[i]);
    };
    if (!skip) {
      const bool edge = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
      if (edge) tile(std::true_type{});
      else tile(std::false_type{});
    }
    wait_dma();
    __syncthreads();
  }

  if (wave_live) {
    const float l_tot = xhalf_sum(l_run);
    const float inv = 1.0f / l_tot;
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int i = 0; i < NDB; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = i * 32 + 8 * rr + 4 * hf;
        u32x2 v = {pack2<BF16>(oacc[i][4 * rr + 0] * inv, oacc[i][4 * rr + 1] * inv),
                   pack2<BF16>(oacc[i][4 * rr + 2] * inv, oacc[i][4 * rr + 3] * inv)};
        buf_store8(ro, (uint32_t)qrow * row_bytes + d0 * 2, v);
      }
    if (hf == 0 && qrow < N) p.lse[((size_t)b * H + h) * N + qrow] = (m_use + fast_log2(l_tot)) * kLn2;
  }
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_t(const FwdParams& p, hipStream_t s) {
  const int nqt = (p.N + kBR - 1) / kBR;
  const dim3 grid((unsigned)(p.B * p.H * nqt));
  hipLaunchKernelGGL((fwd_kernel<BF16, D, CAUSAL>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
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

}  // namespace attn
