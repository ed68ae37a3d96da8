"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

* The oracle: oracle/pkv_oracle.c with tests/c/oracle_sanitize.c, built by gcc with -fsanitize=address,undefined and
  leak checking on; the driver runs every exported oracle function (ragged, empty and partial-block sequences, unit
  lists, splits and combine, the append with skipped slots, varlen, windows, the QKV step, error returns).
* The library's host code: pkv_api.hip, pkv_check.hip and pkv_geometry.hip built by hipcc with the sanitizers on the
  host side only (each -fsanitize after -Xarch_host), the kernel launchers of the other sources replaced by counting
  stubs (tests/c/launch_stubs.hip), linked by the ROCm clang with its sanitizer runtime; tests/c/consumer.c and
  tests/c/host_paths.c then drive the dispatcher over a grid of shapes, the workspace sizing and every argument error,
  and check that no failing call reached a launch.
Any sanitizer report makes the run exit non-zero (halt on the first error, UB included).
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_decode_04_amd", "csrc")
TESTS_C = os.path.join(ROOT, "tests", "c")
ROCM = "/opt/rocm"
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    return r.returncode, r.stdout


def _checked(out):
    lines = [l for l in out.splitlines() if l.startswith(("ok ", "FAIL "))]
    return lines, [l for l in lines if l.startswith("FAIL")]


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_sanitize")
    rc, out = _run([gcc, "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-Wall", "-Werror",
                    os.path.join(ROOT, "oracle", "pkv_oracle.c"), os.path.join(TESTS_C, "oracle_sanitize.c"),
                    "-lpthread", "-lm", "-o", exe])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=300)
    lines, failed = _checked(out)
    assert rc == 0 and not failed and len(lines) >= 20, out


def _asan_runtime_dir():
    hits = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    return os.path.dirname(hits[0]) if hits else None


def test_library_host_paths_under_address_and_undefined_sanitizers(tmp_path):
    rt = _asan_runtime_dir()
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG) and rt):
        pytest.skip("ROCm clang with its sanitizer runtime is not installed")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "--offload-arch=gfx950", "-fPIC",
             "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]
    sources = [os.path.join(CSRC, s) for s in ("pkv_api.hip", "pkv_check.hip", "pkv_geometry.hip")]
    sources.append(os.path.join(TESTS_C, "launch_stubs.hip"))
    procs, objs = [], []
    for src in sources:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC] + flags + ["-c", src, "-o", obj], stdout=subprocess.PIPE,
                                      stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out = p.communicate(timeout=600)[0]
        assert p.returncode == 0, out
    lib = str(tmp_path / "libpkv.so")
    rc, out = _run([CLANG + "++", "-shared", "-fsanitize=address,undefined", "-shared-libasan", "-o", lib] + objs +
                   ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    assert rc == 0, out
    for driver, at_least in (("consumer", 8), ("host_paths", 40)):
        exe = str(tmp_path / driver)
        rc, out = _run([CLANG, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-shared-libasan", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        os.path.join(TESTS_C, driver + ".c"), "-L" + str(tmp_path), "-lpkv",
                        "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath," + rt, "-o", exe])
        assert rc == 0, out
        rc, out = _run([exe], env=ENV, timeout=300)
        lines, failed = _checked(out)
        assert rc == 0 and not failed and len(lines) >= at_least, "%s:\n%s" % (driver, out)
