"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_decode_04_amd.build        # or __graft_entry__.build()

Every HIP translation unit is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns that
it does not know the feature, which is harmless.  After linking, the gfx950
assembly of the kernels is generated once more and searched for packed-FP32
arithmetic (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32), and the kernel
metadata for private (scratch) segments: the build fails if packed-FP32
arithmetic appears or if any kernel spills registers to scratch memory.  The
objects and the assembly are compiled concurrently, then the objects linked.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["pkv_kernels.hip", "pkv_qkv.hip", "pkv_check.hip", "pkv_geometry.hip", "pkv_api.hip"]
# the measurement probe (not part of the attention path): its own library, libpkvprobe.so
PROBE_SRC = os.path.join(PKG, "probe", "pkv_probe.hip")
PROBE_LIB = os.path.join(PKG, "libpkvprobe.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-std=c++17", "-O3", "--offload-arch=" + ARCH, "-fPIC", "-fvisibility=hidden", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]

_PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
_KERNEL_META = re.compile(r"^\s+(?:-\s+)?\.name:\s+(\S+)\s*$|^\s+(?:-\s+)?\.private_segment_fixed_size:\s+(\d+)",
                          re.M)


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    return out


def _check_asm(src: str, tmp: str) -> None:
    """Compile one source to gfx950 assembly and fail on packed-FP32 arithmetic or scratch use."""
    asm = os.path.join(tmp, os.path.basename(src) + ".s")
    _run([HIPCC] + COMMON + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm])
    with open(asm) as f:
        scan_asm(src, f.read())


def scan_asm(src: str, text: str) -> None:
    """Raise if gfx950 assembly text holds packed-FP32 arithmetic or a kernel with a private (scratch) segment."""
    hits = sorted(set(m.group(0) for m in _PACKED_F32.finditer(text)))
    if hits:
        raise RuntimeError("packed-FP32 instructions in %s: %s" % (src, ", ".join(hits)))
    spills, name = [], None
    for m in _KERNEL_META.finditer(text):  # each kernel's .name precedes its segment size
        if m.group(1) is not None:
            name = m.group(1)
        elif name is not None:
            if int(m.group(2)):
                spills.append("%s (%s B)" % (name, m.group(2)))
            name = None
    if spills:
        raise RuntimeError("kernels using scratch memory in %s: %s" % (src, ", ".join(spills)))


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 2 * len(SOURCES)))


def check_no_packed_fp32() -> None:
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(_jobs()) as pool:
        for fut in [pool.submit(_check_asm, src, tmp) for src in SOURCES]:
            fut.result()


def build(verbose: bool = False) -> str:
    """Compile the HIP sources into libpkv.so (always recompiles).

    Each source is compiled to an object, and to assembly for the checks above, in concurrent hipcc processes
    (at most MAX_JOBS, else the CPU count); the objects are then linked into the library.
    """
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(_jobs()) as pool:
        objs = [os.path.join(tmp, src + ".o") for src in SOURCES]
        compiles = [pool.submit(_run, [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj])
                    for src, obj in zip(SOURCES, objs)]
        checks = [pool.submit(_check_asm, src, tmp) for src in SOURCES + [PROBE_SRC]]
        probe_tmp = PROBE_LIB + ".tmp%d" % os.getpid()
        probe = pool.submit(_run, [HIPCC] + COMMON + ["-shared", PROBE_SRC, "-o", probe_tmp])
        out = "\n".join(f.result() for f in compiles)
        lib_tmp = LIB + ".tmp%d" % os.getpid()
        out += _run([HIPCC, "--offload-arch=" + ARCH, "-fPIC", "-shared", "-o", lib_tmp] + objs)
        out += probe.result()
        for f in checks:
            f.result()
    if verbose and out.strip():
        print(out)
    os.replace(lib_tmp, LIB)
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
