#!/usr/bin/env python3
"""Build libkvq.so for gfx950 with hipcc (in-tree, no JIT).

Each .hip translation unit is compiled in parallel, then linked into
packed_cache_attention_amd/libkvq.so.  The library links against the HIP runtime
that ships with PyTorch (same soname as ROCm's), so a process that has imported
torch maps exactly one HIP runtime.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
OUT = os.path.join(PKG, "libkvq.so")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["kvq_api.hip", "kvq_energy_alloc.hip", "kvq_quantize.hip", "kvq_decode.hip", "kvq_decode_mfma.hip", "kvq_prefill.hip", "kvq_rotate.hip",
           "kvq_decode_generic.hip"] + \
    ["kvq_decode_mfma_v%d.hip" % v for v in list(range(1, 9)) + [16]]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         # packed FP32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(PKG), "include")]


def torch_lib_dir():
    try:
        import importlib.util
        spec = importlib.util.find_spec("torch")
        if spec and spec.origin:
            d = os.path.join(os.path.dirname(spec.origin), "lib")
            if os.path.exists(os.path.join(d, "libamdhip64.so")):
                return d
    except Exception:
        pass
    return None


# host code under AddressSanitizer and UBSan (device code unchanged), for checking the
# C ABI's host-side validation on the CPU: libkvq_hostsan.so
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


def _compile(src, extra=(), build_dir=BUILD):
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = [HIPCC] + FLAGS + list(extra) + ["-c", os.path.join(HERE, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    return obj, err


def build(verbose=False, host_sanitize=False):
    extra = HOST_SAN if host_sanitize else []
    build_dir = BUILD + ("_hostsan" if host_sanitize else "")
    out = os.path.join(PKG, "libkvq_hostsan.so") if host_sanitize else OUT
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(int(os.environ.get("MAX_JOBS", "8")), len(SOURCES))) as ex:
        results = list(ex.map(lambda src: _compile(src, extra, build_dir), SOURCES))
    for obj, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    objs = [o for o, _ in results]
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp"] + objs
    if host_sanitize:
        link += ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    tl = torch_lib_dir()
    if tl:
        link += ["-L" + tl, "-Wl,-rpath," + tl]
    subprocess.check_call(link)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, host_sanitize="--host-sanitize" in sys.argv))
