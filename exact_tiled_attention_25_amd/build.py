"""Compile the gfx950 HIP sources in csrc/ into the in-tree shared library libattn.so, and
the measurement probes in probe/ into libattn_probe.so (loaded by bench.py only).

Every call recompiles (the object files are cheap to rebuild and this keeps the library in
step with its sources). Used by ``__graft_entry__.build()`` and ``python -m
exact_tiled_attention_25_amd.build``.
"""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libattn.so")
PROBE_SRC = os.path.join(HERE, "probe", "attn_probe.hip")
PROBE_LIB = os.path.join(HERE, "libattn_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: never emit v_pk_{add,mul,fma}_f32 (hipcc's host pass warns that it does
# not know the feature; that warning is harmless).
# -fno-honor-nans: no kernel input or intermediate is NaN by construction (masked scores are
# -inf, which stays honoured), and it lets fmax chains fuse into v_max3_f32 without the
# operand canonicalisation that IEEE mode otherwise inserts.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fno-honor-nans",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{os.path.join(ROOT, 'include')}"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "hip-link" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, jobs=None):
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    probe_obj = os.path.join(OBJDIR, "attn_probe.o")
    jobs = jobs or min(len(srcs) + 1, os.cpu_count() or 4, 16)
    def flags(src):
        # the C ABI's argument checks must see NaN arguments (-fno-honor-nans would let the
        # compiler assume a float argument is never NaN); it holds no kernels
        return [f for f in FLAGS if f != "-fno-honor-nans"] if src.endswith("attn_api.hip") else FLAGS
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(lambda so: _run([HIPCC, *flags(so[0]), "-c", so[0], "-o", so[1]]),
                           zip(srcs + [PROBE_SRC], objs + [probe_obj])))
    tmp = LIB + ".tmp"
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    outs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", probe_obj, "-o", PROBE_LIB + ".tmp"]))
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    # The host compilation pass can silently drop a kernel's launch stub (for instance when
    # substitution fails in device-only code); the library would then fail to load. Catch
    # that here rather than at first use.
    und = subprocess.run(["nm", "-C", "--undefined-only", tmp], stdout=subprocess.PIPE, text=True).stdout
    missing = [l.strip() for l in und.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs missing from the host objects:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    if verbose:
        for o in outs:
            if o:
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
