"""The C ABI from plain C: tests/c/consumer.c is compiled as C11 against include/pkv.h alone, linked against the
built libpkv.so and run; it exercises the host-only entry points (no device call), so it runs without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "paged_kv_decode_04_amd")


def test_plain_c_consumer(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(LIBDIR, "libpkv.so")):
        pytest.skip("libpkv.so is not built")
    exe = str(tmp_path / "consumer")
    subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "consumer.c"), "-L", LIBDIR, "-lpkv",
                    "-Wl,-rpath," + LIBDIR, "-o", exe], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert len(lines) == 8 and all(l.startswith("ok ") for l in lines), r.stdout
