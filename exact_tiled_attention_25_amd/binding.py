"""Thin ctypes binding of libattn.so (include/attn.h): argument marshalling only.

Each function takes torch tensors that already live on the GPU, checks dtype, shape,
contiguity and device, allocates outputs with torch when the caller passes none, and calls
the C entry point of the same name on the current torch stream. All arithmetic runs in the
HIP kernels; if the library is missing this module raises instead of computing anything.

torch is imported before the library is loaded so that libattn.so binds to the HIP runtime
torch already holds (one runtime per process: shared device memory and streams).
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_BF16, ATTN_FP16 = 0, 1
FP8_BLOCK = 64
EXPORTS = ("attn_fwd", "attn_fwd_gqa", "attn_fwd_varlen", "attn_fwd_splitkv_workspace_bytes",
           "attn_fwd_splitkv", "attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_gqa",
           "attn_bwd_varlen_workspace_bytes", "attn_bwd_varlen", "attn_fp8_quantize",
           "attn_fp8_quantize_per_tensor", "attn_fp8_quantize_rope", "attn_fwd_fp8", "attn_strerror",
           "attn_bwd_noalloc_max_rows", "attn_bwd_noalloc")
_DTYPE_CODE = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_FP16}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load(path=None):
    """Load libattn.so once and declare the C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() first")
    L = ctypes.CDLL(path)
    vp, i, f, sz, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.attn_fwd_gqa.restype = i
    L.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    L.attn_fwd_varlen.restype = i
    L.attn_bwd_varlen_workspace_bytes.argtypes = [i, i]
    L.attn_bwd_varlen_workspace_bytes.restype = sz
    L.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_bwd_varlen.restype = i
    L.attn_fwd_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_fwd_splitkv_workspace_bytes.restype = sz
    L.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    L.attn_fwd_splitkv.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_bwd.restype = i
    L.attn_bwd_noalloc_max_rows.argtypes = []
    L.attn_bwd_noalloc_max_rows.restype = sz
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_bwd_noalloc.restype = i
    L.attn_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_bwd_gqa.restype = i
    for fn in (L.attn_fp8_quantize, L.attn_fp8_quantize_per_tensor):
        fn.argtypes = [vp, vp, vp, i, i, i, i, i, i, u64, vp]
        fn.restype = i
    L.attn_fp8_quantize_rope.argtypes = [vp, vp, vp, i, i, i, i, i, ctypes.c_double, i, u64, vp]
    L.attn_fp8_quantize_rope.restype = i
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, vp, u64, i, vp]
    L.attn_fwd_fp8.restype = i
    L.attn_strerror.argtypes = [i]
    L.attn_strerror.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = L
    return L


def strerror(status):
    return load().attn_strerror(status).decode()


def _check(fn, status):
    if status != 0:
        raise AttnError(fn, status, strerror(status))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _tensor(t, name, shape=None, dtypes=None, device=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def attn_fwd(q, k, v, causal=False, scale=None, o=None, lse=None, stream=None):
    """O, LSE = attention(q, k, v) for [B, N, H, d] bf16/fp16 tensors; LSE is [B, H, N] fp32."""
    _tensor(q, "q", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = q.shape
    _tensor(k, "k", q.shape, (q.dtype,), q.device)
    _tensor(v, "v", q.shape, (q.dtype,), q.device)
    o = torch.empty_like(q) if o is None else _tensor(o, "o", q.shape, (q.dtype,), q.device)
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _tensor(lse, "lse", (B, H, N), (torch.float32,), q.device))
    _check("attn_fwd", load().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                       int(bool(causal)), _default_scale(d, scale), _DTYPE_CODE[q.dtype],
                                       _stream(q, stream)))
    return o, lse


def attn_fwd_gqa(q, k, v, causal=False, scale=None, o=None, lse=None, stream=None):
    """Grouped-query forward: q [B, N, H, d]; k, v [B, N, H_kv, d] with H_kv dividing H."""
    _tensor(q, "q", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = q.shape
    _tensor(k, "k", dtypes=(q.dtype,), device=q.device)
    hkv = k.shape[2] if k.dim() == 4 else 0
    _tensor(k, "k", (B, N, hkv, d), (q.dtype,), q.device)
    _tensor(v, "v", (B, N, hkv, d), (q.dtype,), q.device)
    o = torch.empty_like(q) if o is None else _tensor(o, "o", q.shape, (q.dtype,), q.device)
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _tensor(lse, "lse", (B, H, N), (torch.float32,), q.device))
    _check("attn_fwd_gqa", load().attn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, hkv, N, d,
                                               int(bool(causal)), _default_scale(d, scale), _DTYPE_CODE[q.dtype],
                                               _stream(q, stream)))
    return o, lse


def attn_bwd_gqa(q, k, v, o, lse, do, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None,
                 stream=None):
    """Grouped-query backward: shapes as attn_fwd_gqa; dk, dv have H_kv heads."""
    _tensor(q, "q", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = q.shape
    _tensor(k, "k", dtypes=(q.dtype,), device=q.device)
    hkv = k.shape[2] if k.dim() == 4 else 0
    kv_shape = (B, N, hkv, d)
    _tensor(k, "k", kv_shape, (q.dtype,), q.device)
    _tensor(v, "v", kv_shape, (q.dtype,), q.device)
    for name, t in (("o", o), ("do", do)):
        _tensor(t, name, q.shape, (q.dtype,), q.device)
    _tensor(lse, "lse", (B, H, N), (torch.float32,), q.device)
    dq = torch.empty_like(q) if dq is None else _tensor(dq, "dq", q.shape, (q.dtype,), q.device)
    dk = torch.empty_like(k) if dk is None else _tensor(dk, "dk", kv_shape, (q.dtype,), q.device)
    dv = torch.empty_like(v) if dv is None else _tensor(dv, "dv", kv_shape, (q.dtype,), q.device)
    need = attn_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _tensor(workspace, "workspace", device=q.device)
    _check("attn_bwd_gqa", load().attn_bwd_gqa(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), B, H, hkv, N, d,
        int(bool(causal)), _default_scale(d, scale), _DTYPE_CODE[q.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q, stream)))
    return dq, dk, dv


def _varlen_args(q, k, cu_seqlens, max_seqlen):
    _tensor(q, "q", dtypes=tuple(_DTYPE_CODE))
    if q.dim() != 3:
        raise ValueError("q must be [T, H, d] (packed sequences)")
    T, H, d = q.shape
    _tensor(k, "k", dtypes=(q.dtype,), device=q.device)
    hkv = k.shape[1] if k.dim() == 3 else 0
    _tensor(k, "k", (T, hkv, d), (q.dtype,), q.device)
    _tensor(cu_seqlens, "cu_seqlens", dtypes=(torch.int32,), device=q.device)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of B+1 offsets")
    return T, H, hkv, d, cu_seqlens.numel() - 1, int(max_seqlen)


def attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, causal=False, scale=None, o=None, lse=None, stream=None):
    """Packed variable-length forward: q [T, H, d], k, v [T, H_kv, d], cu_seqlens int32 [B+1]
    on the device, max_seqlen >= every length. Returns O [T, H, d] and LSE [H, T] fp32."""
    T, H, hkv, d, B, ms = _varlen_args(q, k, cu_seqlens, max_seqlen)
    _tensor(v, "v", tuple(k.shape), (q.dtype,), q.device)
    o = torch.empty_like(q) if o is None else _tensor(o, "o", q.shape, (q.dtype,), q.device)
    lse = (torch.empty((H, T), dtype=torch.float32, device=q.device) if lse is None
           else _tensor(lse, "lse", (H, T), (torch.float32,), q.device))
    _check("attn_fwd_varlen", load().attn_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), B, T, ms, H, hkv, d, int(bool(causal)),
        _default_scale(d, scale), _DTYPE_CODE[q.dtype], _stream(q, stream)))
    return o, lse


def attn_bwd_varlen_workspace_bytes(T, H):
    return int(load().attn_bwd_varlen_workspace_bytes(T, H))


def attn_bwd_varlen(q, k, v, o, lse, do, cu_seqlens, max_seqlen, causal=False, scale=None, dq=None, dk=None,
                    dv=None, workspace=None, stream=None):
    """Backward of attn_fwd_varlen (layouts as there)."""
    T, H, hkv, d, B, ms = _varlen_args(q, k, cu_seqlens, max_seqlen)
    _tensor(v, "v", tuple(k.shape), (q.dtype,), q.device)
    for name, t in (("o", o), ("do", do)):
        _tensor(t, name, q.shape, (q.dtype,), q.device)
    _tensor(lse, "lse", (H, T), (torch.float32,), q.device)
    dq = torch.empty_like(q) if dq is None else _tensor(dq, "dq", q.shape, (q.dtype,), q.device)
    dk = torch.empty_like(k) if dk is None else _tensor(dk, "dk", tuple(k.shape), (q.dtype,), q.device)
    dv = torch.empty_like(v) if dv is None else _tensor(dv, "dv", tuple(k.shape), (q.dtype,), q.device)
    if workspace is None:
        workspace = torch.empty(max(attn_bwd_varlen_workspace_bytes(T, H), 1), dtype=torch.uint8, device=q.device)
    _tensor(workspace, "workspace", device=q.device)
    _check("attn_bwd_varlen", load().attn_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_seqlens), B, T,
        ms, H, hkv, d, int(bool(causal)), _default_scale(d, scale), _DTYPE_CODE[q.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q, stream)))
    return dq, dk, dv


def attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits):
    return int(load().attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits))


def attn_fwd_splitkv(q, k, v, num_splits, causal=False, scale=None, o=None, lse=None, workspace=None,
                     stream=None):
    """attn_fwd with each query tile's key range cut into num_splits parts (1..16), merged by
    log-sum-exp; the workspace is allocated here when not given."""
    _tensor(q, "q", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = q.shape
    _tensor(k, "k", q.shape, (q.dtype,), q.device)
    _tensor(v, "v", q.shape, (q.dtype,), q.device)
    o = torch.empty_like(q) if o is None else _tensor(o, "o", q.shape, (q.dtype,), q.device)
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None
           else _tensor(lse, "lse", (B, H, N), (torch.float32,), q.device))
    if workspace is None:
        need = attn_fwd_splitkv_workspace_bytes(B, H, N, d, num_splits)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _tensor(workspace, "workspace", device=q.device)
    _check("attn_fwd_splitkv", load().attn_fwd_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, int(bool(causal)), _default_scale(d, scale),
        _DTYPE_CODE[q.dtype], int(num_splits), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(q, stream)))
    return o, lse


def attn_bwd_workspace_bytes(B, H, N, d):
    return int(load().attn_bwd_workspace_bytes(B, H, N, d))


def attn_bwd(q, k, v, o, lse, do, causal=False, scale=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None):
    """dQ, dK, dV of sum(dO o O) by LSE recomputation; tensors as in attn_fwd."""
    _tensor(q, "q", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _tensor(t, name, q.shape, (q.dtype,), q.device)
    _tensor(lse, "lse", (B, H, N), (torch.float32,), q.device)
    dq = torch.empty_like(q) if dq is None else _tensor(dq, "dq", q.shape, (q.dtype,), q.device)
    dk = torch.empty_like(q) if dk is None else _tensor(dk, "dk", q.shape, (q.dtype,), q.device)
    dv = torch.empty_like(q) if dv is None else _tensor(dv, "dv", q.shape, (q.dtype,), q.device)
    need = attn_bwd_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _tensor(workspace, "workspace", device=q.device)
    _check("attn_bwd", load().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                                       _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)),
                                       _default_scale(d, scale), _DTYPE_CODE[q.dtype], _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(q, stream)))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, do, causal=False, scale=None, dq=None, dk=None, dv=None, stream=None):
    """attn_bwd without a workspace: the library's fixed device scratch holds D (B*H*N rows at
    most attn_bwd_noalloc_max_rows()). Allocates nothing when dq, dk, dv are given."""
    _tensor(q, "q", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _tensor(t, name, q.shape, (q.dtype,), q.device)
    _tensor(lse, "lse", (B, H, N), (torch.float32,), q.device)
    dq = torch.empty_like(q) if dq is None else _tensor(dq, "dq", q.shape, (q.dtype,), q.device)
    dk = torch.empty_like(q) if dk is None else _tensor(dk, "dk", q.shape, (q.dtype,), q.device)
    dv = torch.empty_like(q) if dv is None else _tensor(dv, "dv", q.shape, (q.dtype,), q.device)
    _check("attn_bwd_noalloc", load().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do),
                                                       _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(bool(causal)),
                                                       _default_scale(d, scale), _DTYPE_CODE[q.dtype],
                                                       _stream(q, stream)))
    return dq, dk, dv


def attn_bwd_noalloc_max_rows():
    return int(load().attn_bwd_noalloc_max_rows())


def attn_fp8_quantize(x, rotate, hadamard_seed=0, x8=None, descale=None, stream=None, per_tensor=False):
    """e4m3 codes [B, N, H, d] (uint8) and fp32 descales [B, H, ceil(N/64)] of x: one descale
    per 64-row block, or with per_tensor=True one descale for all of x (in every entry)."""
    _tensor(x, "x", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = x.shape
    nblk = (N + FP8_BLOCK - 1) // FP8_BLOCK
    x8 = (torch.empty(x.shape, dtype=torch.uint8, device=x.device) if x8 is None
          else _tensor(x8, "x8", x.shape, (torch.uint8,), x.device))
    descale = (torch.empty((B, H, nblk), dtype=torch.float32, device=x.device) if descale is None
               else _tensor(descale, "descale", (B, H, nblk), (torch.float32,), x.device))
    name = "attn_fp8_quantize_per_tensor" if per_tensor else "attn_fp8_quantize"
    _check(name, getattr(load(), name)(_ptr(x), _ptr(x8), _ptr(descale), B, H, N, d,
                                       _DTYPE_CODE[x.dtype], int(bool(rotate)),
                                       int(hadamard_seed) & (2 ** 64 - 1), _stream(x, stream)))
    return x8, descale


def attn_fp8_quantize_per_tensor(x, rotate, hadamard_seed=0, x8=None, descale=None, stream=None):
    """attn_fp8_quantize with one descale for the whole tensor."""
    return attn_fp8_quantize(x, rotate, hadamard_seed, x8, descale, stream, per_tensor=True)


def attn_fp8_quantize_rope(x, rotate, hadamard_seed=0, rope_base=10000.0, x8=None, descale=None, stream=None):
    """Fused RoPE (row n of each batch at position n) + optional Hadamard rotation + 64-row
    block quantisation of x [B, N, H, d]: e4m3 codes and fp32 descales [B, H, ceil(N/64)]."""
    _tensor(x, "x", dtypes=tuple(_DTYPE_CODE))
    B, N, H, d = x.shape
    nblk = (N + FP8_BLOCK - 1) // FP8_BLOCK
    x8 = (torch.empty(x.shape, dtype=torch.uint8, device=x.device) if x8 is None
          else _tensor(x8, "x8", x.shape, (torch.uint8,), x.device))
    descale = (torch.empty((B, H, nblk), dtype=torch.float32, device=x.device) if descale is None
               else _tensor(descale, "descale", (B, H, nblk), (torch.float32,), x.device))
    _check("attn_fp8_quantize_rope",
           load().attn_fp8_quantize_rope(_ptr(x), _ptr(x8), _ptr(descale), B, H, N, d, _DTYPE_CODE[x.dtype],
                                         float(rope_base), int(bool(rotate)),
                                         int(hadamard_seed) & (2 ** 64 - 1), _stream(x, stream)))
    return x8, descale


def attn_fwd_fp8(q8, k8, v8, descale_q, descale_k, descale_v, causal=False, scale=None,
                 hadamard_seed=0, out_dtype=torch.bfloat16, o=None, lse=None, stream=None):
    """FP8 forward: O (out_dtype) and LSE (fp32) from e4m3 codes and per-block descales."""
    _tensor(q8, "q8", dtypes=(torch.uint8,))
    B, N, H, d = q8.shape
    nblk = (N + FP8_BLOCK - 1) // FP8_BLOCK
    _tensor(k8, "k8", q8.shape, (torch.uint8,), q8.device)
    _tensor(v8, "v8", q8.shape, (torch.uint8,), q8.device)
    for name, t in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        _tensor(t, name, (B, H, nblk), (torch.float32,), q8.device)
    if out_dtype not in _DTYPE_CODE:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float16")
    o = (torch.empty(q8.shape, dtype=out_dtype, device=q8.device) if o is None
         else _tensor(o, "o", q8.shape, (out_dtype,), q8.device))
    lse = (torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if lse is None
           else _tensor(lse, "lse", (B, H, N), (torch.float32,), q8.device))
    _check("attn_fwd_fp8", load().attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, H, N, d,
                                               int(bool(causal)), _default_scale(d, scale), _ptr(descale_q),
                                               _ptr(descale_k), _ptr(descale_v), int(hadamard_seed) & (2 ** 64 - 1),
                                               _DTYPE_CODE[out_dtype], _stream(q8, stream)))
    return o, lse
