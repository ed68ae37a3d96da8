"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_decode_04_amd.build        # or __graft_entry__.build()

Every HIP translation unit is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host pass warns that
it does not know the feature, which is harmless.  After linking, the gfx950
assembly of the kernels is generated once more and searched for packed-FP32
arithmetic (v_pk_add_f32 / v_pk_mul_f32 / v_pk_fma_f32), and the kernel
metadata for private (scratch) segments: the build fails if packed-FP32
arithmetic appears or if any kernel spills registers to scratch memory.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpkv.so")
SOURCES = ["pkv_kernels.hip", "pkv_qkv.hip", "pkv_check.hip", "pkv_api.hip"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-std=c++17", "-O3", "--offload-arch=" + ARCH, "-fPIC", "-fvisibility=hidden", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]

_PACKED_F32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")
_KERNEL_META = re.compile(r"^\s+\.name:\s+(\S+)\s*$|^\s+\.private_segment_fixed_size:\s+(\d+)", re.M)


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (r.returncode, " ".join(cmd), out))
    return out


def check_no_packed_fp32() -> None:
    with tempfile.TemporaryDirectory() as tmp:
        for src in SOURCES:
            asm = os.path.join(tmp, src + ".s")
            _run([HIPCC] + COMMON + ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", asm])
            with open(asm) as f:
                text = f.read()
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


def build(verbose: bool = False) -> str:
    """Compile the HIP sources into libpkv.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + COMMON + ["-shared", "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    out = _run(cmd)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    check_no_packed_fp32()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
