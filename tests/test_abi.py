"""C-ABI contract checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    from exact_tiled_attention_25_amd import binding
    assert set(_declared_functions()) == set(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_strerror_covers_every_status(lib):
    msgs = {s: lib.attn_strerror(s).decode() for s in range(7)}
    assert msgs[0] == "success"
    assert len(set(msgs.values())) == 7
    assert lib.attn_strerror(99).decode() == "unknown status"


def test_workspace_size(lib):
    assert lib.attn_bwd_workspace_bytes(2, 16, 8192, 128) == 2 * 16 * 8192 * 8
    assert lib.attn_bwd_workspace_bytes(0, 16, 8192, 128) == 0


@pytest.mark.parametrize("args,status", [
    (dict(d=100), 2), (dict(d=32), 2), (dict(B=-1), 1), (dict(N=-5), 1),
    (dict(scale=float("nan")), 1), (dict(scale=-0.1), 1), (dict(scale=float("inf")), 1),
    (dict(dtype=7), 1), (dict(B=0), 0), (dict(N=0), 0), (dict(H=0), 0),
    (dict(N=2 ** 30), 2),
])
def test_fwd_argument_validation_without_device(lib, args, status):
    a = dict(B=1, H=1, N=16, d=64, causal=0, scale=0.125, dtype=0)
    a.update(args)
    # null tensor pointers: every case above must be decided before pointers or the device matter
    got = lib.attn_fwd(None, None, None, None, None, a["B"], a["H"], a["N"], a["d"], a["causal"],
                       a["scale"], a["dtype"], None)
    assert got == status


def test_null_pointers_rejected(lib):
    assert lib.attn_fwd(None, None, None, None, None, 1, 1, 16, 64, 0, 0.125, 0, None) == 1
    assert lib.attn_bwd(None, None, None, None, None, None, None, None, None, 1, 1, 16, 64, 0, 0.125, 0,
                        None, 0, None) == 1
    assert lib.attn_fp8_quantize(None, None, None, 1, 1, 16, 64, 0, 1, 0, None) == 1
    assert lib.attn_fp8_quantize_per_tensor(None, None, None, 1, 1, 16, 64, 0, 1, 0, None) == 1
    assert lib.attn_fp8_quantize_rope(None, None, None, 1, 1, 16, 64, 0, 10000.0, 1, 0, None) == 1
    # RoPE base: finite and above 1, checked before pointers or the device
    for base in (1.0, 0.5, -10000.0, float("nan"), float("inf")):
        assert lib.attn_fp8_quantize_rope(None, None, None, 1, 1, 16, 64, 0, base, 1, 0, None) == 1
    assert lib.attn_fp8_quantize_rope(None, None, None, 1, 1, 16, 96, 0, 10000.0, 1, 0, None) == 2
    assert lib.attn_fp8_quantize_rope(None, None, None, 0, 1, 16, 64, 0, 10000.0, 1, 0, None) == 0
    assert lib.attn_fwd_gqa(None, None, None, None, None, 1, 4, 2, 16, 64, 0, 0.125, 0, None) == 1
    assert lib.attn_fwd_gqa(None, None, None, None, None, 1, 4, 3, 16, 64, 0, 0.125, 0, None) == 1
    assert lib.attn_fwd_gqa(None, None, None, None, None, 1, 4, 0, 16, 64, 0, 0.125, 0, None) == 1
    assert lib.attn_bwd_gqa(None, None, None, None, None, None, None, None, None, 1, 4, 2, 16, 64, 0, 0.125, 0,
                            None, 0, None) == 1
    assert lib.attn_bwd_gqa(None, None, None, None, None, None, None, None, None, 1, 6, 4, 16, 64, 0, 0.125, 0,
                            None, 0, None) == 1
    assert lib.attn_fwd_varlen(None, None, None, None, None, None, 2, 100, 64, 4, 2, 64, 0, 0.125, 0, None) == 1
    assert lib.attn_fwd_varlen(None, None, None, None, None, None, -1, 100, 64, 4, 2, 64, 0, 0.125, 0, None) == 1
    cu = (ctypes.c_int * 3)(0, 40, 100)  # only checked for null on the host
    assert lib.attn_fwd_varlen(None, None, None, None, None, cu, 2, 100, 64, 4, 2, 96, 0, 0.125, 0, None) == 2
    assert lib.attn_fwd_varlen(None, None, None, None, None, cu, 2, 100, 64, 4, 3, 64, 0, 0.125, 0, None) == 1
    assert lib.attn_fwd_varlen(None, None, None, None, None, None, 2, 0, 64, 4, 2, 64, 0, 0.125, 0, None) == 0
    assert lib.attn_bwd_varlen(None, None, None, None, None, None, None, None, None, None, 2, 100, 64, 4, 3, 64, 0,
                               0.125, 0, None, 0, None) == 1
    assert lib.attn_bwd_varlen_workspace_bytes(100, 4) == 3200
    assert lib.attn_fwd_splitkv(None, None, None, None, None, 1, 1, 16, 64, 0, 0.125, 0, 2, None, 0, None) == 1
    assert lib.attn_fwd_splitkv(None, None, None, None, None, 1, 1, 16, 64, 0, 0.125, 0, 0, None, 0, None) == 1
    assert lib.attn_fwd_splitkv(None, None, None, None, None, 1, 1, 16, 96, 0, 0.125, 0, 2, None, 0, None) == 2
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 2, 100, 64, 3) == 3 * 2 * 100 * 65 * 4
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 2, 100, 64, 17) == 0
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 2, 100, 96, 2) == 0
    assert lib.attn_fp8_quantize_per_tensor(None, None, None, 1, 1, 16, 100, 0, 1, 0, None) == 2
    assert lib.attn_fwd_fp8(None, None, None, None, None, 1, 1, 16, 64, 0, 0.125, None, None, None, 0, 0,
                            None) == 1


def test_bwd_noalloc_limits_without_device(lib):
    """The no-allocation backward checks its arguments like attn_bwd, then its fixed scratch
    limit (B*H*N rows), all before any device access."""
    assert lib.attn_bwd_noalloc_max_rows() == 1 << 22
    nul = [None] * 9
    assert lib.attn_bwd_noalloc(*nul, 1, 1, 16, 64, 0, 0.125, 0, None) == 1
    assert lib.attn_bwd_noalloc(*nul, 0, 1, 16, 64, 0, 0.125, 0, None) == 0
    assert lib.attn_bwd_noalloc(*nul, 1, 1, 16, 96, 0, 0.125, 0, None) == 2
    fake = [ctypes.c_void_p(4096)] * 9   # never dereferenced: the size check fails first
    assert lib.attn_bwd_noalloc(*fake, 2, 16, (1 << 17) + 1, 64, 0, 0.125, 0, None) == 6
    assert lib.attn_bwd_noalloc(*fake, 1, 1, 16, 64, 0, float("nan"), 0, None) == 1


def test_non_finite_scale_rejected_with_pointers(lib):
    """NaN and infinite scales are rejected even when every pointer is set (the checks are not
    masked by the null-pointer check, and the compiler may not assume arguments are NaN-free)."""
    fake = [ctypes.c_void_p(4096)] * 9
    for bad in (float("nan"), float("inf"), -1.0):
        assert lib.attn_fwd(*fake[:5], 1, 1, 16, 64, 0, bad, 0, None) == 1
        assert lib.attn_bwd(*fake, 1, 1, 16, 64, 0, bad, 0, None, 0, None) == 1
        assert lib.attn_bwd_noalloc(*fake, 1, 1, 16, 64, 0, bad, 0, None) == 1
        assert lib.attn_fwd_fp8(*fake[:5], 1, 1, 16, 64, 0, bad, *fake[:3], 0, 0, None) == 1
    for base in (float("nan"), float("inf")):
        assert lib.attn_fp8_quantize_rope(*fake[:3], 1, 1, 16, 64, 0, base, 1, 0, None) == 1


def test_probe_library_exports_its_probes():
    """The measurement probes bench.py reports (matrix-core ceiling, VALU costs, LDS read
    rates, fp32 atomic rate) are built into their own library and load without a device."""
    path = os.path.join(ROOT, "exact_tiled_attention_25_amd", "libattn_probe.so")
    if not os.path.exists(path):
        pytest.skip("libattn_probe.so is not built")
    probe = ctypes.CDLL(path)
    for name in ("probe_mfma", "probe_mfma_once", "probe_valu", "probe_lds", "probe_atomic"):
        assert hasattr(probe, name), name
