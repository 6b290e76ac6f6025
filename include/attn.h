/* attn.h - exact tiled attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libattn.so. Every tensor pointer is DEVICE memory owned by the caller. The
 * library allocates nothing, never synchronises the host, and enqueues all its work on the
 * caller's stream in call order. Calls return after the launch; a status other than
 * ATTN_OK means nothing was enqueued (argument and device errors) or the launch itself
 * failed (ATTN_ELAUNCH). No C++ exception crosses this interface.
 *
 * Shapes and layout (the same for every entry point):
 *   Q, K, V, O, dO, dQ, dK, dV : [B][N][H][d] contiguous ("token-major", row pitch H*d),
 *                                 element type given by `dtype` (bf16 or fp16).
 *   LSE                         : [B][H][N] fp32, natural-log log-sum-exp of each query row.
 *   FP8 tensors                 : [B][N][H][d] OCP e4m3 bytes (E4M3FN: bias 7, max 448).
 *   FP8 descales                : [B][H][ceil(N/64)] fp32; real value = e4m3 value * descale
 *                                 of the 64-row block the row lies in.
 * Sizes: B, H, N >= 0 (a zero size is an empty problem and returns ATTN_OK doing nothing);
 * d in {64, 128, 256}; N need not be a multiple of any tile size. The causal mask lets
 * query i see key j iff j <= i. `scale` must be finite and >= 0 (usually 1/sqrt(d)).
 *
 * Sources: the pages "FlashAttention-3: Hopper Asynchrony and FP8 Attention" (Symbol Map,
 * Deep Dive, Putting It Together) and "FlashAttention 3 Hardware Acceleration: Hopper GPU
 * Strategies for Long-Context Enterprise Inference Optimization" (FP8 sections).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_FP8_BLOCK 64 /* rows per FP8 quantisation block */

typedef enum { ATTN_BF16 = 0, ATTN_FP16 = 1 } attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,        /* null pointer, negative size, non-finite or negative scale, bad enum */
  ATTN_EUNSUPPORTED = 2,  /* d not in {64,128,256}, or a size whose indices overflow 32 bits */
  ATTN_EWORKSPACE = 3,    /* workspace missing or smaller than attn_bwd_workspace_bytes() */
  ATTN_ELAUNCH = 4,       /* the HIP runtime rejected a kernel launch */
  ATTN_EDEVICE = 5,       /* the current device is not gfx950 */
  ATTN_ETOOLARGE = 6      /* beyond the fixed scratch of attn_bwd_noalloc */
} attn_status_t;

/* A hipStream_t passed as an opaque pointer; NULL means the null stream. */
typedef void* attn_stream_t;

/* Forward exact attention: O = softmax(scale * Q K^T [+ causal mask]) V and
 * LSE_i = m_i + ln(l_i) (Symbol Map; "Putting It Together", epilogue row: O is divided by
 * l and only O and L are written). O and LSE are overwritten. */
attn_status_t attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, int causal, float scale,
                       attn_dtype_t dtype, attn_stream_t stream);

/* Grouped-query forward: the key/value heads are shared by groups of query heads (the
 * enterprise post, "Runtime Kernel Selection", lists grouped query attention among the
 * supported patterns; it gives no formula). q, o: [B][N][H][d]; k, v: [B][N][H_kv][d] with
 * 1 <= H_kv and H % H_kv == 0; query head h attends to key/value head h / (H / H_kv).
 * Otherwise as attn_fwd (attn_fwd is the case H_kv = H). ATTN_EINVAL for a bad H_kv. */
attn_status_t attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int H_kv, int N, int d, int causal, float scale,
                           attn_dtype_t dtype, attn_stream_t stream);

/* Variable-length batches (packed): B sequences of lengths cu_seqlens[b+1] - cu_seqlens[b],
 * stored back to back. q, o: [T][H][d]; k, v: [T][H_kv][d] (H_kv dividing H, grouped as in
 * attn_fwd_gqa); lse: [H][T] fp32. cu_seqlens is DEVICE memory, B+1 int32 offsets with
 * 0 = cu[0] <= cu[1] <= ... <= cu[B] = T; max_seqlen >= every length (it sizes the grid).
 * Each sequence is an independent attention (causal: token i of a sequence sees tokens 0..i
 * of the same sequence); the enterprise post lists variable-length handling among the
 * kernel's forthcoming features ("GPU Compatibility and Enablement Matrix"). The offsets are
 * not read on the host: offsets outside [0, T] or lengths above max_seqlen are clamped, so
 * they give unspecified results but no access outside the tensors. Errors as attn_fwd, plus
 * ATTN_EINVAL for negative sizes or a null cu_seqlens. */
attn_status_t attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                              const int* cu_seqlens, int B, int T, int max_seqlen, int H, int H_kv,
                              int d, int causal, float scale, attn_dtype_t dtype,
                              attn_stream_t stream);

/* Bytes of device workspace attn_bwd_varlen needs: the per-row fp32 pairs (L log2 e,
 * D = rowsum(dO o O)), [H][T][2]. */
size_t attn_bwd_varlen_workspace_bytes(int T, int H);

/* Backward of attn_fwd_varlen: layouts as there; dq [T][H][d], dk, dv [T][H_kv][d]. */
attn_status_t attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              const int* cu_seqlens, int B, int T, int max_seqlen, int H, int H_kv,
                              int d, int causal, float scale, attn_dtype_t dtype, void* workspace,
                              size_t workspace_bytes, attn_stream_t stream);

/* Bytes of device workspace attn_fwd_splitkv needs: per part, O_s fp32 [B][H][N][d] and
 * L_s fp32 [B][H][N] (num_splits * B*H*N*(d+1) * 4 bytes). 0 for invalid arguments. */
size_t attn_fwd_splitkv_workspace_bytes(int B, int H, int N, int d, int num_splits);

/* Forward exact attention with the key range split: the results of attn_fwd (up to
 * rounding), for problems too small to fill the GPU one query tile per workgroup (short N,
 * few heads). Each query tile's key tiles are cut into num_splits contiguous parts
 * (1 <= num_splits <= 16) that separate workgroups process; part s yields O_s = O/l and
 * L_s over its keys, and a merge forms L = log sum_s exp(L_s) and O = sum_s exp(L_s - L) O_s
 * (the log-sum-exp state of the online softmax, Symbol Map: m_i, l_i, L_i; the same merge
 * that joins sequence shards in ring attention, enterprise post "Million-Token Context
 * Windows"). Parts with no key for a row (causal) are skipped. `workspace` must hold
 * attn_fwd_splitkv_workspace_bytes(...) bytes; contents on entry are ignored, on return
 * unspecified. Errors as attn_fwd, plus ATTN_EINVAL for num_splits out of range and
 * ATTN_EWORKSPACE. */
attn_status_t attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int d, int causal, float scale,
                               attn_dtype_t dtype, int num_splits, void* workspace,
                               size_t workspace_bytes, attn_stream_t stream);

/* Bytes of device workspace attn_bwd needs: the per-row fp32 pairs (L log2 e,
 * D = rowsum(dO o O)), [B][H][N][2]. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d);

/* Backward pass with LSE recomputation (Deep Dive "Backward warp specialization": S and P
 * are recomputed from L, then dP, dS, dV, dK and dQ are formed). Inputs are the forward's
 * Q, K, V, O, LSE and the output gradient dO; dQ, dK, dV are overwritten (not accumulated).
 * `workspace` must hold attn_bwd_workspace_bytes(B,H,N,d) bytes; its contents on entry
 * are ignored and on return unspecified. The result is deterministic (no atomics). */
attn_status_t attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       int B, int H, int N, int d, int causal, float scale,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                       attn_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): attn_bwd with no workspace argument.
 * Same arguments, kernels, results (bit for bit) and errors as attn_bwd; the per-row
 * statistics (two fp32 a row) live in a fixed library-owned device array of
 * attn_bwd_noalloc_max_rows() rows (4 Mi rows, 32 MiB, held by each GPU the library runs on
 * until the process ends). B*H*N above that limit returns ATTN_ETOOLARGE. Nothing is allocated, also not on
 * the first call on a device (which looks up the array's device address). Every call on
 * one GPU shares that array: calls that may overlap on the same GPU (different streams,
 * host threads) race and must be ordered by the caller. ATTN_ELAUNCH if the array's device
 * address cannot be obtained. */
size_t attn_bwd_noalloc_max_rows(void);
attn_status_t attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int B, int H, int N, int d, int causal, float scale,
                               attn_dtype_t dtype, attn_stream_t stream);

/* Grouped-query backward: shapes as attn_fwd_gqa; dq [B][N][H][d], dk and dv
 * [B][N][H_kv][d]. A key/value head's dK and dV are the sums of the gradients through each of
 * its H / H_kv query heads, formed in one workgroup per 128 keys (deterministic, no atomics).
 * Workspace as attn_bwd (attn_bwd_workspace_bytes(B, H, N, d)); attn_bwd is H_kv = H. */
attn_status_t attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           int B, int H, int H_kv, int N, int d, int causal, float scale,
                           attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                           attn_stream_t stream);

/* FP8 block quantisation ("FP8 accuracy controls": one fp32 scale per block; incoherent
 * processing multiplies Q and K by the same orthogonal M = diag(s) H_d / sqrt(d)).
 * x [B][N][H][d] (dtype) -> x8 e4m3 codes and descale [B][H][ceil(N/64)].
 * rotate != 0 applies M with signs s_t = (top bit of SplitMix64 output t for
 * `hadamard_seed`) ? -1 : +1; rotate = 0 quantises x as is (use it for V).
 * descale = fp32(amax/448) of the rotated block (1 for an all-zero block); codes are
 * round-to-nearest-even of value/descale, saturated to +-448. */
attn_status_t attn_fp8_quantize(const void* x, uint8_t* x8, float* descale,
                                int B, int H, int N, int d, attn_dtype_t dtype,
                                int rotate, uint64_t hadamard_seed, attn_stream_t stream);

/* FP8 quantisation with ONE scale for the whole tensor: the per-tensor baseline that
 * block quantisation is measured against (explainer, "FP8 accuracy controls"; the
 * enterprise post "FlashAttention 3 Hardware Acceleration", sections "FP8 Accumulation"
 * and "FP8 Validation": block scales replace a single scale for the entire tensor).
 * Same arguments, rotation and encoding as attn_fp8_quantize; descale = fp32(amax/448)
 * with amax over every (rotated) element of x (1 for an all-zero tensor), and that value is
 * written to all B*H*ceil(N/64) descale entries, so attn_fwd_fp8 takes the result as is.
 * B*H*ceil(N/64) must stay below 2^31. Runs three kernels on `stream`; the descale array
 * holds intermediate values between them. */
attn_status_t attn_fp8_quantize_per_tensor(const void* x, uint8_t* x8, float* descale,
                                           int B, int H, int N, int d, attn_dtype_t dtype,
                                           int rotate, uint64_t hadamard_seed,
                                           attn_stream_t stream);

/* Fused prologue: rotary position embedding, then the random-sign Hadamard rotation, then
 * 64-row block quantisation, in one pass over x ("FP8 accuracy controls": the Hadamard
 * transform can be fused with rotary embedding; the enterprise post names the same fusion).
 * The pages do not define the embedding; it is RoPE as in Su et al., "RoFormer" (2021): the
 * row at position n (its index 0 .. N-1 within its batch) has each pair of dims (2i, 2i+1)
 * turned by the angle n * rope_base^(-2i/d): (a, b) -> (a cos - b sin, a sin + b cos).
 * Apply it to Q and K with the same seed (attention then sees the scores of RoPE attention;
 * V takes attn_fp8_quantize with rotate = 0). Arguments, codes and descales otherwise as
 * attn_fp8_quantize. rope_base must be finite and > 1 (ATTN_EINVAL otherwise; 10000 is the
 * usual value). Angles are reduced modulo 2 pi in fp64; sine, cosine and the pair rotation
 * are fp32. */
attn_status_t attn_fp8_quantize_rope(const void* x, uint8_t* x8, float* descale,
                                     int B, int H, int N, int d, attn_dtype_t dtype,
                                     double rope_base, int rotate, uint64_t hadamard_seed,
                                     attn_stream_t stream);

/* FP8 forward attention ("FP8 layout conformance", "FP8 accuracy controls"):
 * O = softmax(scale * Qh Kh^T [+ mask]) Vh with Xh = e4m3(X8) * descale_X per 64-row block.
 * Q8 and K8 must have been rotated with the same seed (or both not at all); because the
 * rotation is orthogonal the scores do not depend on it, and `hadamard_seed` is carried
 * only to describe the inputs. The probabilities are rounded to e4m3 for the P V product,
 * scaled by 64 * dv/dv_max (dv the V descale of the key's block, dv_max the head's largest);
 * the epilogue undoes that factor exactly. O is written in `out_dtype`, LSE in fp32 (natural log).
 * Every descale must be finite and >= 0 (the quantisers write positive ones); a zero descale
 * is a block of zeros, and a head whose V descales are all zero gets O = 0. Negative or
 * non-finite descales give undefined results (no access leaves the tensors). */
attn_status_t attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                           void* o, float* lse, int B, int H, int N, int d, int causal,
                           float scale, const float* descale_q, const float* descale_k,
                           const float* descale_v, uint64_t hadamard_seed,
                           attn_dtype_t out_dtype, attn_stream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* attn_strerror(attn_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
