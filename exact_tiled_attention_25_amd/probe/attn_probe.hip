// Measurement probes for the roofline denominators (not part of the attention library):
//  * probe_mfma: a dependency-free loop of v_mfma_f32_32x32x16_bf16 or
//    v_mfma_f32_32x32x64_f8f6f4 (8 independent accumulators per wave, operands held in
//    registers, no memory traffic) on random or on all-zero operands. The sustained rate
//    on random data is the practical ceiling of the matrix cores: under full MFMA load the
//    chip lowers its clock, and more so the more bits toggle.
//  * probe_valu: cycles per wave64 instruction of v_exp_f32 (the softmax exponential),
//    v_fma_f32, v_cvt_pk_fp8_f32 and v_cvt_pk_bf16_f32 on one or two waves per SIMD (16
//    independent registers per wave, so latency is hidden), from s_memtime, and the shader
//    clock during the loop from the ratio of s_memtime to the fixed-rate s_memrealtime
//    (100 MHz).
//  * probe_atomic: fp32 global atomic adds (or plain stores) of 64 x 128 tiles into a
//    [2][8192][16][128] fp32 accumulator, one workgroup per (head, 128-key tile) walking
//    nqt query tiles: the traffic a key-outer backward would make to accumulate dQ
//    across its key tiles, to price that design against recomputing S and dP in a
//    separate query-outer pass.
//  * probe_lds: LDS read throughput with eight waves per CU, for the two operand reads the
//    attention kernels issue: ds_read_b128 of 16-byte row chunks at the K-tile pitch
//    (2d + 16 bytes at d = 128) and ds_read_b64_tr_b16 at the V-tile pitch (2d + 64), both
//    conflict-free by construction, eight reads in flight per wave, timed with s_memtime.
// Built into libattn_probe.so, loaded only by bench.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {   // integer hash (lowbias32)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}
__device__ __forceinline__ float unit(uint32_t h) {   // uniform in [-1, 1)
  return (float)(int)h * 0x1p-31f;
}

template <int KIND>   // 0: bf16 32x32x16, 1: fp8 (e4m3) 32x32x64
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters, int zero) {
  using Op = typename std::conditional<KIND == 0, bf16x8, i32x8>::type;
  const uint32_t gid = blockIdx.x * 256 + threadIdx.x;
  Op a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h0 = mix(gid * 64 + k * 16 + e), h1 = mix(~(gid * 64 + k * 16 + e));
      if constexpr (KIND == 0) {
        a[k][e] = (__bf16)(zero ? 0.f : unit(h0));
        b[k][e] = (__bf16)(zero ? 0.f : unit(h1));
      } else {
        int pa = __builtin_amdgcn_cvt_pk_fp8_f32(unit(h0), unit(mix(h0)), 0, false);
        pa = __builtin_amdgcn_cvt_pk_fp8_f32(unit(mix(h0 + 1)), unit(mix(h0 + 2)), pa, true);
        int pb = __builtin_amdgcn_cvt_pk_fp8_f32(unit(h1), unit(mix(h1)), 0, false);
        pb = __builtin_amdgcn_cvt_pk_fp8_f32(unit(mix(h1 + 1)), unit(mix(h1 + 2)), pb, true);
        a[k][e] = zero ? 0 : pa;
        b[k][e] = zero ? 0 : pb;
      }
    }
  }
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (KIND == 0)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k & 3], b[(k + 1) & 3], acc[k], 0, 0, 0);
      else
        acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[k & 3], b[(k + 1) & 3], acc[k], 0, 0, 0, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[gid] = s;
}

constexpr int kValuRegs = 16;

template <int OP>   // 0: v_exp_f32, 1: v_fma_f32, 2: v_cvt_pk_fp8_f32, 3: v_cvt_pk_bf16_f32
__global__ __launch_bounds__(512) void valu_probe_kernel(unsigned long long* out, int iters) {
  // 96 KiB of LDS per workgroup: one workgroup (4 or 8 waves: one or two per SIMD) per CU
  __shared__ char pad[96 * 1024];
  if (iters < 0) pad[threadIdx.x] = 1;
  float x[kValuRegs];
#pragma unroll
  for (int k = 0; k < kValuRegs; ++k) x[k] = -1.0f + 0.01f * (float)(threadIdx.x % 7 + k);
  const float m = 0.999f, c = 0.0001f;
  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t0 = __builtin_readcyclecounter();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kValuRegs; ++k) {
      if constexpr (OP == 0) asm volatile("v_exp_f32 %0, %0" : "+v"(x[k]));
      else if constexpr (OP == 1) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[k]) : "v"(m), "v"(c));
      else if constexpr (OP == 2) asm volatile("v_cvt_pk_fp8_f32 %0, %0, %1" : "+v"(x[k]) : "v"(c));
      else asm volatile("v_cvt_pk_bf16_f32 %0, %0, %1" : "+v"(x[k]) : "v"(c));
    }
  }
  const unsigned long long t1 = __builtin_readcyclecounter();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kValuRegs; ++k) s += x[k];
  const int wave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  if (threadIdx.x % 64 == 0) {
    out[3 * wave] = t1 - t0;
    out[3 * wave + 1] = r1 - r0;
    out[3 * wave + 2] = (unsigned long long)__float_as_uint(s);
  }
}

// One MFMA on given operands (one wave): fp8 32x32x64 (kind 0) or bf16 32x32x16 (kind 1);
// a, b: 64 lanes x 32 bytes (fp8) or 16 bytes (bf16) in the MFMA's register layout; c, d: 64
// lanes x 16 floats. Used to read how the matrix core adds its products and its accumulator.
typedef float f32x4p __attribute__((ext_vector_type(4)));
// kind 2: fp8 16x16x128 (a, b: 32 bytes per lane; c, d: first 4 floats per lane); kind 3:
// fp8 32x32x64 with the E8M0 scale code `sb` on B (and 127, i.e. 1.0, on A).
__global__ __launch_bounds__(64) void mfma_once_kernel(int kind, const uint32_t* a, const uint32_t* b,
                                                       const float* c, float* d, int sb) {
  const int l = threadIdx.x;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = c[l * 16 + r];
  if (kind == 2) {
    i32x8 x, y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = (int)a[l * 8 + e];
      y[e] = (int)b[l * 8 + e];
    }
    f32x4p r4 = {acc[0], acc[1], acc[2], acc[3]};
    r4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, r4, 0, 0, 0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = r4[r];
  } else if (kind == 3) {
    i32x8 x, y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = (int)a[l * 8 + e];
      y[e] = (int)b[l * 8 + e];
    }
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, 0, 0, 0, 127, 0, sb);
  } else if (kind == 0) {
    i32x8 x, y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = (int)a[l * 8 + e];
      y[e] = (int)b[l * 8 + e];
    }
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, acc, 0, 0, 0, 0, 0, 0);
  } else {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v xa = {a[l * 4], a[l * 4 + 1], a[l * 4 + 2], a[l * 4 + 3]};
    const u32x4v xb = {b[l * 4], b[l * 4 + 1], b[l * 4 + 2], b[l * 4 + 3]};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa), __builtin_bit_cast(bf16x8, xb), acc,
                                                  0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) d[l * 16 + r] = acc[r];
}

// MODE 0: global_atomic_add_f32 (no return), 1: plain store. Workgroup w: head w / 64
// (b = head / 16, h = head % 16), 128-key tile w % 64; wave rows 16 per query tile.
template <int MODE>
__global__ __launch_bounds__(256) void atomic_probe_kernel(float* ws, int nqt) {
  const int head = blockIdx.x / 64;
  const int b = head / 16, h = head % 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int qt = 0; qt < nqt; ++qt) {
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
      const int row = qt * 64 + wave * 16 + (i >> 1);   // < 64 nqt <= 8192
      const int d = (i & 1) * 64 + lane;                // < 128
      float* p = ws + (((size_t)b * 8192 + row) * 16 + h) * 128 + d;
      if (MODE == 0) __hip_atomic_fetch_add(p, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *p = 1.0f;
    }
  }
}

// KIND 0: ds_read_b128, 1: ds_read_b64_tr_b16. 80 KiB of LDS (one workgroup per CU), 8
// waves; out[block * 8 + wave] = s_memtime cycles of the wave's loop.
template <int KIND>
__global__ __launch_bounds__(512, 1) void lds_probe_kernel(unsigned long long* out, int iters) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(1024))) char buf[81920];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 81920 / 4; i += 512) ((uint32_t*)buf)[i] = mix((uint32_t)i);
  __syncthreads();
  const int i16 = lane & 15, grp = lane >> 4, hf = grp >> 1;
  // row chunks: rows l%32 at pitch 272, chunk l/32; transposed: rows 4hf + i16/4 at pitch
  // 320, dims 16 (grp%2) + 4 (i16%4). Largest byte read: 3*20480 + 8448 + 224 + 8704 + 16
  // (rows) and 3*20480 + 2296 + 448 + 5120 + 8 (transposed), both inside the 80 KiB.
  const int off = KIND == 0 ? (lane & 31) * 272 + (lane >> 5) * 16
                            : (4 * hf + (i16 >> 2)) * 320 + (16 * (grp & 1) + 4 * (i16 & 3)) * 2;
  const char* base = buf + (wave & 3) * 20480 + off;
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if (KIND == 0) {
      u32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) v[r] = *(const u32x4*)(base + r * 32 + (it & 1) * 8704);
#pragma unroll
      for (int r = 0; r < 8; ++r) asm volatile("" ::"v"(v[r]));
    } else {
      s16x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + r * 64 + (it & 1) * 5120));
#pragma unroll
      for (int r = 0; r < 8; ++r) asm volatile("" ::"v"(v[r]));
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) out[blockIdx.x * 8 + wave] = t1 - t0;
}

}  // namespace

extern "C" {

// 256 workgroups (one per CU) of 8 waves, each wave iters x 8 reads; out: 2048 uint64 of
// device memory (per-wave cycles). Synchronises the stream. Returns a hipError_t.
int probe_lds(int kind, int iters, void* stream, unsigned long long* out) {
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0) hipLaunchKernelGGL(lds_probe_kernel<0>, dim3(256), dim3(512), 0, s, out, iters);
  else hipLaunchKernelGGL(lds_probe_kernel<1>, dim3(256), dim3(512), 0, s, out, iters);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  return (int)err;
}

// 2048 workgroups (32 heads x 64 key tiles), each adding (mode 0) or storing (mode 1) nqt
// 64 x 128 fp32 tiles (1 <= nqt <= 128) into ws, which holds 2 * 8192 * 16 * 128 floats of
// device memory; *ms = elapsed time on `stream` (HIP events). Returns a hipError_t.
int probe_atomic(int mode, float* ws, int nqt, void* stream, float* ms) {
  if (nqt < 1 || nqt > 128 || (mode != 0 && mode != 1)) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return (int)hipErrorUnknown;
  hipError_t err = hipEventRecord(e0, s);
  if (err == hipSuccess) {
    if (mode == 0) hipLaunchKernelGGL(atomic_probe_kernel<0>, dim3(2048), dim3(256), 0, s, ws, nqt);
    else hipLaunchKernelGGL(atomic_probe_kernel<1>, dim3(2048), dim3(256), 0, s, ws, nqt);
    err = hipGetLastError();
  }
  if (err == hipSuccess) err = hipEventRecord(e1, s);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  if (err == hipSuccess) err = hipEventElapsedTime(ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return (int)err;
}

// One wave, one MFMA (see mfma_once_kernel); synchronises the stream.
int probe_mfma_once(int kind, const void* a, const void* b, const float* c, float* d, int sb, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  hipLaunchKernelGGL(mfma_once_kernel, dim3(1), dim3(64), 0, s, kind, (const uint32_t*)a, (const uint32_t*)b, c, d,
                     sb);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  return (int)err;
}


// Runs `blocks` workgroups of 4 waves, each wave `iters` x 8 MFMAs; *ms = elapsed time on
// `stream` (HIP events). out: blocks * 256 floats of device memory. Returns a hipError_t.
int probe_mfma(int kind, int zero_data, int blocks, int iters, void* stream, float* out, float* ms) {
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return (int)hipErrorUnknown;
  hipError_t err = hipEventRecord(e0, s);
  if (err == hipSuccess) {
    if (kind == 0) hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters, zero_data);
    else hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters, zero_data);
    err = hipGetLastError();
  }
  if (err == hipSuccess) err = hipEventRecord(e1, s);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  if (err == hipSuccess) err = hipEventElapsedTime(ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return (int)err;
}

// 256 workgroups (one per CU) of 4 * waves_per_simd waves (1 or 2); out: 3 * 1024 *
// waves_per_simd uint64 of device memory, per wave (s_memtime delta, s_memrealtime delta,
// checksum). Synchronises the stream.
int probe_valu(int op, int iters, int waves_per_simd, void* stream, unsigned long long* out) {
  hipStream_t s = (hipStream_t)stream;
  if (waves_per_simd != 1 && waves_per_simd != 2) return (int)hipErrorInvalidValue;
  const dim3 blk(256 * waves_per_simd);
  if (op == 0) hipLaunchKernelGGL(valu_probe_kernel<0>, dim3(256), blk, 0, s, out, iters);
  else if (op == 1) hipLaunchKernelGGL(valu_probe_kernel<1>, dim3(256), blk, 0, s, out, iters);
  else if (op == 2) hipLaunchKernelGGL(valu_probe_kernel<2>, dim3(256), blk, 0, s, out, iters);
  else hipLaunchKernelGGL(valu_probe_kernel<3>, dim3(256), blk, 0, s, out, iters);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess) err = hipStreamSynchronize(s);
  return (int)err;
}

}  // extern "C"
