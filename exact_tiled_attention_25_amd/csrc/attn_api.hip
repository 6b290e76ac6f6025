// C ABI of libattn.so: argument validation, device check and dispatch to the kernels.
// Nothing here allocates, synchronises or touches tensor contents on the host.
#include <atomic>
#include <cmath>
#include <cstring>

#include "../../include/attn.h"
#include "attn_launch.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

attn_status_t check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_EDEVICE;
  if (dev < kMaxDevices) {
    const int st = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (st == 1) return ATTN_OK;
    if (st == 2) return ATTN_EDEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_EDEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? ATTN_OK : ATTN_EDEVICE;
}

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

// Fixed device scratch of the no-allocation backward: the backward's per-row statistics
// (L log2 e, D = rowsum(dO o O)), two fp32 per (batch, head, row). In host code `scratch`
// only names the symbol; its device address on each GPU comes from hipGetSymbolAddress
// (each device holds its own copy until the process ends).
constexpr size_t kNoAllocMaxRows = (size_t)1 << 22;
constexpr size_t kBwdStatBytes = 2 * sizeof(float);   // workspace bytes per (batch, head, row)
__device__ __align__(256) float scratch[2 * kNoAllocMaxRows];   // 32 MiB
std::atomic<float*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first call there.
attn_status_t scratch_address(float** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_EDEVICE;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return ATTN_ELAUNCH;
    p = (float*)q;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return ATTN_OK;
}

// Sizes shared by every entry point. Byte offsets inside one batch slice are 32-bit
// (buffer addressing), so a batch slice of a 16-bit tensor must stay below 2^31 bytes.
attn_status_t check_sizes(int B, int H, int N, int d, bool* empty) {
  if (B < 0 || H < 0 || N < 0) return ATTN_EINVAL;
  if (!supported_d(d)) return ATTN_EUNSUPPORTED;
  *empty = (B == 0 || H == 0 || N == 0);
  if (*empty) return ATTN_OK;
  const double slice = (double)N * H * d * 2.0;
  if (slice >= 2147483648.0 - 65536.0 * H * d) return ATTN_EUNSUPPORTED;
  if ((double)B * H * ((N + 127) / 128) >= 2147483647.0) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

// (This file is built with NaNs honoured, unlike the kernels: see build.py.)
bool bad_scale(float scale) { return !std::isfinite(scale) || scale < 0.f; }

attn_status_t launched(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ELAUNCH; }

constexpr double kLog2e = 1.4426950408889634074;

// SplitMix64 (Steele, Lea and Flood, 2014): output t of the generator seeded with `seed`.
uint64_t splitmix64_output(uint64_t seed, uint64_t t) {
  uint64_t z = seed + (t + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

}  // namespace

extern "C" {

// Variable-length batches: cu (device, B+1 offsets) and T (total tokens); otherwise null, 0.
static attn_status_t fwd_common(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int Hkv, int N, int d, int causal, float scale,
                                attn_dtype_t dtype, attn_stream_t stream, const int* cu = nullptr,
                                int T = 0) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_EINVAL;
  if (bad_scale(scale)) return ATTN_EINVAL;
  bool empty = false;
  attn_status_t st = check_sizes(B, H, N, d, &empty);
  if (st != ATTN_OK) return st;
  if (Hkv < 1 || (H > 0 && H % Hkv != 0)) return ATTN_EINVAL;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
  if ((st = check_device()) != ATTN_OK) return st;
  attn::FwdParams p{q, k, v, o, lse, B, H, N, (float)(scale * kLog2e), Hkv, cu, T};
  (void)hipGetLastError();
  return launched(attn::launch_fwd(dtype == ATTN_BF16, d, causal != 0, p, (hipStream_t)stream));
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, int causal, float scale,
                       attn_dtype_t dtype, attn_stream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, H > 0 ? H : 1, N, d, causal, scale, dtype, stream);
}

attn_status_t attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int H_kv, int N, int d, int causal, float scale,
                           attn_dtype_t dtype, attn_stream_t stream) {
  return fwd_common(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, dtype, stream);
}

// Checks of a variable-length batch that need no device access (the offsets live there).
static attn_status_t check_varlen(const int* cu, int B, int T, int max_seqlen, int H, bool* empty) {
  if (B < 0 || T < 0 || max_seqlen < 0 || H < 0) return ATTN_EINVAL;
  if (B > 0 && T > 0 && max_seqlen > 0 && H > 0 && !cu) return ATTN_EINVAL;
  if ((double)T * H * 4 >= 2147483647.0 * 8) return ATTN_EUNSUPPORTED;   // per-row kernels' grids
  *empty = B == 0 || T == 0 || max_seqlen == 0 || H == 0;
  return ATTN_OK;
}

attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens, int B, int T, int max_seqlen, int H, int H_kv,
                              int d, int causal, float scale, attn_dtype_t dtype,
                              attn_stream_t stream) {
  bool empty = false;
  attn_status_t st = check_varlen(cu_seqlens, B, T, max_seqlen, H, &empty);
  if (st != ATTN_OK) return st;
  if (!supported_d(d)) return ATTN_EUNSUPPORTED;
  if (empty) return (H_kv < 1 || (H > 0 && H % H_kv != 0)) ? ATTN_EINVAL : ATTN_OK;
  return fwd_common(q, k, v, o, lse, B, H, H_kv, max_seqlen, d, causal, scale, dtype, stream,
                    cu_seqlens, T);
}

size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits) {
  if (B <= 0 || H <= 0 || N <= 0 || !supported_d(d) || num_splits < 1 || num_splits > 16) return 0;
  return (size_t)num_splits * B * H * N * (size_t)(d + 1) * sizeof(float);
}

attn_status_t attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int d, int causal, float scale,
                               attn_dtype_t dtype, int num_splits, void* workspace,
                               size_t workspace_bytes, attn_stream_t stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_EINVAL;
  if (bad_scale(scale)) return ATTN_EINVAL;
  if (num_splits < 1 || num_splits > 16) return ATTN_EINVAL;
  bool empty = false;
  attn_status_t st = check_sizes(B, H, N, d, &empty);
  if (st != ATTN_OK || empty) return st;
  // grids: one workgroup per (query tile, head, batch, part); merge: 8 or more rows each
  if ((double)B * H * ((N + 127) / 128) * num_splits >= 2147483647.0 || (double)B * H * N / 8 >= 2147483647.0)
    return ATTN_EUNSUPPORTED;
  if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
  if (!workspace || workspace_bytes < attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits))
    return ATTN_EWORKSPACE;
  if ((st = check_device()) != ATTN_OK) return st;
  float* ws = (float*)workspace;
  attn::FwdParams p{q, k, v, o, lse, B, H, N, (float)(scale * kLog2e), H, nullptr, 0, num_splits, ws,
                    ws + (size_t)num_splits * B * H * N * d};
  (void)hipGetLastError();
  return launched(attn::launch_fwd_splitkv(dtype == ATTN_BF16, d, causal != 0, p, (hipStream_t)stream));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)B * H * N * kBwdStatBytes;
}

static attn_status_t bwd_common(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                int B, int H, int Hkv, int N, int d, int causal, float scale,
                                attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                attn_stream_t stream, const int* cu = nullptr, int T = 0) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_EINVAL;
  if (bad_scale(scale)) return ATTN_EINVAL;
  bool empty = false;
  attn_status_t st = check_sizes(B, H, N, d, &empty);
  if (st != ATTN_OK) return st;
  if (Hkv < 1 || (H > 0 && H % Hkv != 0)) return ATTN_EINVAL;
  if (empty) return ATTN_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_EINVAL;
  const size_t need = cu ? attn_bwd_varlen_workspace_bytes(T, H) : attn_bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return ATTN_EWORKSPACE;
  if ((st = check_device()) != ATTN_OK) return st;
  attn::BwdParams p{q, k, v, o, lse, dout, dq, dk, dv, (float*)workspace, B, H, N, scale,
                    (float)(scale * kLog2e), Hkv, cu, T};
  (void)hipGetLastError();
  return launched(attn::launch_bwd(dtype == ATTN_BF16, d, causal != 0, p, (hipStream_t)stream));
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int B, int H, int N, int d, int causal, float scale,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                       attn_stream_t stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, H, H > 0 ? H : 1, N, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream);
}

size_t attn_bwd_varlen_workspace_bytes(int T, int H) {
  if (T <= 0 || H <= 0) return 0;
  return (size_t)T * H * kBwdStatBytes;
}

attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              const int* cu_seqlens, int B, int T, int max_seqlen, int H, int H_kv,
                              int d, int causal, float scale, attn_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, attn_stream_t stream) {
  bool empty = false;
  attn_status_t st = check_varlen(cu_seqlens, B, T, max_seqlen, H, &empty);
  if (st != ATTN_OK) return st;
  if (!supported_d(d)) return ATTN_EUNSUPPORTED;
  if (empty) return (H_kv < 1 || (H > 0 && H % H_kv != 0)) ? ATTN_EINVAL : ATTN_OK;
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, max_seqlen, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream, cu_seqlens, T);
}

size_t attn_bwd_noalloc_max_rows(void) { return kNoAllocMaxRows; }

attn_status_t attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int H, int N, int d, int causal, float scale,
                               attn_dtype_t dtype, attn_stream_t stream) {
  // the argument checks of attn_bwd, then the size limit, then the device and its scratch
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_EINVAL;
  if (bad_scale(scale)) return ATTN_EINVAL;
  bool empty = false;
  attn_status_t st = check_sizes(B, H, N, d, &empty);
  if (st != ATTN_OK || empty) return st;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_EINVAL;
  if ((double)B * H * N > (double)kNoAllocMaxRows) return ATTN_ETOOLARGE;
  if ((st = check_device()) != ATTN_OK) return st;
  float* ws = nullptr;
  if ((st = scratch_address(&ws)) != ATTN_OK) return st;
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, d, causal, scale, dtype, ws,
                    kNoAllocMaxRows * kBwdStatBytes, stream);
}

attn_status_t attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int H_kv, int N, int d, int causal, float scale,
                           attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                           attn_stream_t stream) {
  return bwd_common(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, causal, scale, dtype,
                    workspace, workspace_bytes, stream);
}

static attn_status_t fp8_quantize(const void* x, uint8_t* x8, float* descale, int B, int H, int N,
                                  int d, attn_dtype_t dtype, int rotate, uint64_t hadamard_seed,
                                  bool per_tensor, attn_stream_t stream, double rope_base = 0.0) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_EINVAL;
  const bool rope = rope_base != 0.0;
  if (rope && !(std::isfinite(rope_base) && rope_base > 1.0)) return ATTN_EINVAL;
  bool empty = false;
  attn_status_t st = check_sizes(B, H, N, d, &empty);
  if (st != ATTN_OK || empty) return st;
  // one workgroup per 64-row block (and, per tensor, one int count of all blocks)
  if ((double)B * H * ((N + 63) / 64) >= 2147483647.0) return ATTN_EUNSUPPORTED;
  if (!x || !x8 || !descale) return ATTN_EINVAL;
  if ((st = check_device()) != ATTN_OK) return st;
  attn::Fp8QuantParams p{x, x8, descale, B, H, N, rotate != 0, {0, 0, 0, 0, 0, 0, 0, 0}, per_tensor ? 1 : 0,
                         rope ? 1 : 0, rope ? std::log2(rope_base) : 0.0};
  if (rotate)
    for (int t = 0; t < d; ++t)
      if (splitmix64_output(hadamard_seed, (uint64_t)t) >> 63) p.neg[t >> 5] |= 1u << (t & 31);
  (void)hipGetLastError();
  return launched(attn::launch_fp8_quantize(dtype == ATTN_BF16, d, p, (hipStream_t)stream));
}

attn_status_t attn_fp8_quantize(const void* x, uint8_t* x8, float* descale,
                                int B, int H, int N, int d, attn_dtype_t dtype,
                                int rotate, uint64_t hadamard_seed, attn_stream_t stream) {
  return fp8_quantize(x, x8, descale, B, H, N, d, dtype, rotate, hadamard_seed, false, stream);
}

attn_status_t attn_fp8_quantize_per_tensor(const void* x, uint8_t* x8, float* descale,
                                           int B, int H, int N, int d, attn_dtype_t dtype,
                                           int rotate, uint64_t hadamard_seed, attn_stream_t stream) {
  return fp8_quantize(x, x8, descale, B, H, N, d, dtype, rotate, hadamard_seed, true, stream);
}

attn_status_t attn_fp8_quantize_rope(const void* x, uint8_t* x8, float* descale,
                                     int B, int H, int N, int d, attn_dtype_t dtype,
                                     double rope_base, int rotate, uint64_t hadamard_seed,
                                     attn_stream_t stream) {
  if (!(std::isfinite(rope_base) && rope_base > 1.0)) return ATTN_EINVAL;
  return fp8_quantize(x, x8, descale, B, H, N, d, dtype, rotate, hadamard_seed, false, stream, rope_base);
}

attn_status_t attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                           void* o, float* lse, int B, int H, int N, int d, int causal,
                           float scale, const float* descale_q, const float* descale_k,
                           const float* descale_v, uint64_t hadamard_seed,
                           attn_dtype_t out_dtype, attn_stream_t stream) {
  (void)hadamard_seed;  // scores do not depend on the (shared, orthogonal) rotation
  if (out_dtype != ATTN_BF16 && out_dtype != ATTN_FP16) return ATTN_EINVAL;
  if (bad_scale(scale)) return ATTN_EINVAL;
  bool empty = false;
  attn_status_t st = check_sizes(B, H, N, d, &empty);
  if (st != ATTN_OK || empty) return st;
  if (!q8 || !k8 || !v8 || !o || !lse || !descale_q || !descale_k || !descale_v) return ATTN_EINVAL;
  if ((st = check_device()) != ATTN_OK) return st;
  attn::Fp8FwdParams p{q8, k8, v8, descale_q, descale_k, descale_v, o, lse, B, H, N,
                       (float)(scale * kLog2e)};
  (void)hipGetLastError();
  return launched(attn::launch_fwd_fp8(out_dtype == ATTN_BF16, d, causal != 0, p, (hipStream_t)stream));
}

const char* attn_strerror(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument (null pointer, negative size, bad scale or enum)";
    case ATTN_EUNSUPPORTED: return "unsupported shape (head dim must be 64, 128 or 256; batch slice below 2 GiB)";
    case ATTN_EWORKSPACE: return "workspace missing or too small (see attn_*_workspace_bytes)";
    case ATTN_ELAUNCH: return "kernel launch failed";
    case ATTN_EDEVICE: return "current device is not an MI355X-class gfx950 GPU";
    case ATTN_ETOOLARGE: return "problem larger than the fixed scratch of a no-allocation entry point";
  }
  return "unknown status";
}

}  // extern "C"
