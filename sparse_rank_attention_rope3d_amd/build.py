"""Build libslr.so (HIP, gfx950 only) in-tree with hipcc.

    python -m sparse_rank_attention_rope3d_amd.build

Each source compiles to an object under csrc/_build/, then they link into
sparse_rank_attention_rope3d_amd/libslr.so. Packed fp32 VALU instructions are
disabled for the device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libslr.so")
SOURCES = ["k_rope.hip", "k_select.hip", "k_lowrank.hip", "k_flash.hip", "k_backward.hip", "slr_api.cpp"]
# the bench's memory-hierarchy read probe, a library of its own (not part of the layer's ABI)
PROBE_OUT = os.path.join(PKG, "libslr_probe.so")
PROBE_SOURCES = ["probe_stream.hip"]
# the same library with the host code of the C ABI (argument checks, workspace
# layout, launch sequence) built under AddressSanitizer and UBSan, for the CPU
# ABI tests; the kernels' objects are the regular ones
HOSTSAN_OUT = os.path.join(PKG, "libslr_hostsan.so")
HOSTSAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                 "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, obj: str, extra) -> None:
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; nothing else is expected
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def _link(objs, out: str, extra=()) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(extra=(), jobs: int = 8) -> str:
    bdir = os.path.join(CSRC, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], list(extra)), zip(srcs, objs)))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    # host-sanitized variant: slr_api.cpp again with the sanitizers on its host side only
    san_obj = os.path.join(bdir, "slr_api_hostsan.o")
    flags = [f for f in FLAGS if f != "-O3"]
    cmd = [HIPCC, *flags, *HOSTSAN_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, "slr_api.cpp"), "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized slr_api.cpp:\n{r.stdout}\n{r.stderr}")
    kernel_objs = [o for o, src in zip(objs, srcs) if src in SOURCES and src != "slr_api.cpp"]
    _link([san_obj, *kernel_objs], HOSTSAN_OUT,
          extra=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"])
    return OUT


if __name__ == "__main__":
    print(build(sys.argv[1:]))
