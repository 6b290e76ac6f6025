// Forward exact attention for gfx950: one workgroup per (query tile, head, batch).
//
// Method (page "FlashAttention-3: Hopper Asynchrony and FP8 Attention"): the query tile
// Q_i stays resident while K_j, V_j tiles stream past it (Symbol Map); each tile gives
// S = Q_i K_j^T, the online softmax keeps a running row maximum m_i and sum l_i, P~ V_j is
// added to the output numerator, and the epilogue divides by l_i and stores O_i and
// L_i = m_i + log(l_i) ("Putting It Together", steps 2-7).
//
// gfx950 design (the Hopper producer/consumer, TMA and WGMMA machinery is prior art only):
//  * 4 waves x 32 query rows = 128 rows per workgroup; key tiles of BC = 64 (d = 64: 128).
//  * K and V tiles are fetched with coalesced 16-byte buffer loads one tile ahead into
//    registers and written to the other half of a two-stage LDS ring, so one barrier per
//    tile separates the ring stages. Rows past N load as zeros (buffer range check).
//  * Scores are produced transposed, S^T = K Q^T (MFMA 32x32x16): each lane then owns ONE
//    query row (column l%32 of the accumulator) and 16 keys of each 32-key block, so the
//    row maximum is an in-lane reduction plus one permlane32 swap, and the row sum stays a
//    per-lane partial until the epilogue.
//  * The score accumulator is the B operand of O^T += V^T P^T without any lane exchange:
//    accumulator r of lane half hf is key 8*(r/4) + 4*hf + r%4, so the MFMA's 8 k-slots
//    (16*cc + 8*hf + s) meet keys whose index has bits 2 and 3 swapped. V is therefore
//    stored transposed in LDS ([d][key], key contiguous, as MFMA operands must be) at
//    position swap23(key); its 16-byte groups are XOR-swizzled by row to spread LDS banks.
//  * Online softmax in the exp2 domain (scores scaled by scale*log2 e with one FMA), and
//    a lazy rescale: the reference maximum only moves (and O, l are only rescaled) when a
//    row's maximum grows by more than 2^8, decided per wave with a ballot. Any reference
//    value gives the same exact O and L; this one keeps P~ <= 256 and skips most rescales.
//  * Causal: tiles past the diagonal are never loaded; longest query tiles launch first;
//    waves whose rows all precede a tile skip its math.
//  * Block ids are remapped so that all query tiles of a head run on one XCD (shared L2).
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

template <int D> struct FwdCfg;
template <> struct FwdCfg<64> { static constexpr int BC = 128; };
template <> struct FwdCfg<128> { static constexpr int BC = 64; };
template <> struct FwdCfg<256> { static constexpr int BC = 64; };

constexpr int kWaves = 4;
constexpr int kQW = 32;                  // query rows per wave
constexpr int kBR = kWaves * kQW;        // query rows per workgroup
constexpr float kTau = 8.0f;             // lazy-rescale threshold (log2 units)
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ int swap01(int x) { return (x & ~3) | ((x & 1) << 1) | ((x >> 1) & 1); }

// XOR swizzle of the 16-byte groups of V^T row d (NG groups per row).
template <int NG>
__device__ __forceinline__ int vswz(int d) {
  if constexpr (NG == 8) return (d ^ (d >> 3)) & 7;
  else return (d ^ (d >> 4)) & 15;
}

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdParams p) {
  constexpr int BC = FwdCfg<D>::BC;
  constexpr int KP = D * 2 + 16;         // K tile row pitch (bytes), padded against bank conflicts
  constexpr int KBYTES = BC * KP;
  constexpr int VP = BC * 2;             // V^T row pitch (bytes)
  constexpr int VBYTES = D * VP;
  constexpr int STAGE = KBYTES + VBYTES;
  constexpr int NG = BC / 8;
  constexpr int KIT = BC * D / 8 / 256;  // 16-byte K loads per thread per tile
  constexpr int VIT = BC * D / 32 / 256; // (4 keys x 8 dims) V items per thread per tile
  constexpr int NKB = BC / 32;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  static_assert(KIT >= 1 && VIT >= 1 && (BC * D / 8) % 256 == 0 && (BC * D / 32) % 256 == 0, "tile split");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

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

  // Q^T operand: lane holds query q0 + l32, dims 16*ks + 8*hf .. +7.
  u32x4 qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qreg[ks] = buf_load16(rq, (uint32_t)(q0 + l32) * row_bytes + (16 * ks + 8 * hf) * 2);

  const int kend = CAUSAL ? min(N, (qt + 1) * kBR) : N;
  const int nkt = (kend + BC - 1) / BC;

  u32x4 kreg[KIT];
  u32x4 vreg[VIT][4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = tid + 256 * it, c8 = i % (D / 8), kr = i / (D / 8);
      kreg[it] = buf_load16(rk, (uint32_t)(k0 + kr) * row_bytes + c8 * 16);
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int i = tid + 256 * it, c8 = i % (D / 8), kg = i / (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) vreg[it][r] = buf_load16(rv, (uint32_t)(k0 + 4 * kg + r) * row_bytes + c8 * 16);
    }
  };
  auto store_tile = [&](int stage) {
    char* ks = smem + stage * STAGE;
    char* vs = ks + KBYTES;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int i = tid + 256 * it, c8 = i % (D / 8), kr = i / (D / 8);
      *(u32x4*)(ks + kr * KP + c8 * 16) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int i = tid + 256 * it, c8 = i % (D / 8), kg = i / (D / 8);
      const int pg = swap01(kg);           // keys 4kg..4kg+3 sit at positions 4pg..4pg+3
      const int g = pg >> 1, off8 = (pg & 1) * 8;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = vreg[it][0][w], a1 = vreg[it][1][w], a2 = vreg[it][2][w], a3 = vreg[it][3][w];
        const int d0 = c8 * 8 + 2 * w;
        u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *(u32x2*)(vs + d0 * VP + ((g ^ vswz<NG>(d0)) & (NG - 1)) * 16 + off8) = lo;
        *(u32x2*)(vs + (d0 + 1) * VP + ((g ^ vswz<NG>(d0 + 1)) & (NG - 1)) * 16 + off8) = hi;
      }
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const bool wave_live = q0 < N;
  const int qrow = q0 + l32;
  const float c = p.c;

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
          const u32x4 a = *(const u32x4*)(ks + (kb * 32 + l32) * KP + (16 * kk + 8 * hf) * 2);
          s[kb] = mfma32x16<BF16>(a, qreg[kk], s[kb]);
        }
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
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = xhalf_max(mx);
      const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
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
          if (edge) e = (s[kb][r] == -INFINITY) ? 0.f : e;
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
      for (int i = 0; i < NDB; ++i) {
        const int d = i * 32 + l32;
        const char* vrow = vs + d * VP;
        const int sw = vswz<NG>(d);
#pragma unroll
        for (int cidx = 0; cidx < BC / 16; ++cidx) {
          const u32x4 a = *(const u32x4*)(vrow + (((2 * cidx + hf) ^ sw) & (NG - 1)) * 16);
          oacc[i] = mfma32x16<BF16>(a, pk[cidx], oacc[i]);
        }
      }
    }
    if (more) store_tile((j + 1) & 1);
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
