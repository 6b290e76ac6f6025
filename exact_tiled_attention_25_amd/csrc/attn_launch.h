// Internal launch interface between the C ABI (attn_api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N;
  float c;  // softmax scale * log2(e): scores are exponentiated with exp2
  int Hkv;  // key/value heads (divides H); query head h reads key/value head h / (H / Hkv)
  // variable-length batches: cu_seqlens [B+1] (device) or null; with it, N is the longest
  // sequence, tensors are packed [T][heads][d] and LSE is [H][T]
  const int* cu;
  int T;
  // split-KV only: S = splits part slots per query tile; a query tile with n key tiles
  // uses ceil(n / split_tiles) of them (split_tiles = ceil(ceil(N/64) / S)); the per-part
  // results O_s = O/l (fp32 [S][B][H][N][d]) and L_s (fp32 [S][B][H][N]; -inf: no keys of
  // the row in the part). A query tile with one part writes o and lse directly.
  int splits;
  float* o_part;
  float* lse_part;
  int split_tiles;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  // workspace: per row the pair (L log2 e, D = rowsum(dO o O)), fp32 [B][H][N][2]
  float* stats;
  int B, H, N;
  float scale;
  float c;  // scale * log2(e)
  int Hkv;  // key/value heads (divides H); dK, dV are [B][N][Hkv][d]
  const int* cu;  // variable-length batches as in FwdParams (then stats is [H][T][2])
  int T;
};

struct Fp8QuantParams {
  const void* x;
  uint8_t* x8;
  float* descale;
  int B, H, N;
  int rotate;
  uint32_t neg[8];  // bit t set: dim t of the random sign vector is -1 (d <= 256)
  int per_tensor;   // one descale for the whole tensor instead of one per 64-row block
  int rope;         // rotary position embedding of each row (position = row index) first
  double rope_log2_base;  // log2 of the RoPE base: pair i turns by n * base^(-2i/d)
};

struct Fp8FwdParams {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* dq;
  const float* dk;
  const float* dv;
  void* o;
  float* lse;
  int B, H, N;
  float c;
};

hipError_t launch_fwd(bool bf16, int d, bool causal, const FwdParams& p, hipStream_t s);
// the split-KV forward, then the merge of its parts into p.o and p.lse
hipError_t launch_fwd_splitkv(bool bf16, int d, bool causal, const FwdParams& p, hipStream_t s);
hipError_t launch_bwd(bool bf16, int d, bool causal, const BwdParams& p, hipStream_t s);
hipError_t launch_fp8_quantize(bool bf16, int d, const Fp8QuantParams& p, hipStream_t s);
hipError_t launch_fwd_fp8(bool out_bf16, int d, bool causal, const Fp8FwdParams& p, hipStream_t s);

}  // namespace attn
