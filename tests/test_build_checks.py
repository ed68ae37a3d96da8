"""Host tests of the build's assembly checks (packed-FP32 arithmetic and scratch segments fail the build)."""
import os
import shutil
import tempfile

import pytest

from paged_kv_decode_04_amd import build

CLEAN = """
\tv_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]
\tv_add_f32_e32 v1, v2, v3
amdhsa.kernels:
  - .agpr_count:     0
    .name:           pkv_kernel_a
    .private_segment_fixed_size: 0
  - .agpr_count:     4
    .name:           pkv_kernel_b
    .private_segment_fixed_size: 0
"""


def test_clean_assembly_passes():
    build.scan_asm("clean.hip", CLEAN)


@pytest.mark.parametrize("op", ["v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"])
def test_packed_fp32_arithmetic_fails(op):
    text = CLEAN.replace("v_add_f32_e32 v1, v2, v3", "%s v[0:1], v[2:3], v[4:5]" % op)
    with pytest.raises(RuntimeError, match=op):
        build.scan_asm("packed.hip", text)


def test_other_packed_ops_pass():
    # packed f16 and packed moves are not the packed-FP32 arithmetic the build rules out
    build.scan_asm("pk16.hip", CLEAN + "\tv_pk_add_f16 v1, v2, v3\n\tv_pk_mov_b32 v[0:1], v[2:3], v[4:5]\n")


def test_a_kernel_with_scratch_fails_and_is_named():
    text = CLEAN.replace("pkv_kernel_b\n    .private_segment_fixed_size: 0",
                         "pkv_kernel_b\n    .private_segment_fixed_size: 48")
    with pytest.raises(RuntimeError, match=r"pkv_kernel_b \(48 B\)"):
        build.scan_asm("spill.hip", text)


def test_a_kernel_entry_opening_with_its_name_is_read_too():
    text = "amdhsa.kernels:\n  - .name:           pkv_kernel_c\n    .private_segment_fixed_size: 16\n"
    with pytest.raises(RuntimeError, match=r"pkv_kernel_c \(16 B\)"):
        build.scan_asm("first.hip", text)


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not installed")
def test_real_assembly_of_the_check_kernels_passes_and_names_them():
    with tempfile.TemporaryDirectory() as tmp:
        build._check_asm("pkv_check.hip", tmp)
        with open(os.path.join(tmp, "pkv_check.hip.s")) as f:
            names = [m.group(1) for m in build._KERNEL_META.finditer(f.read()) if m.group(1)]
    assert any("check_indices_kernel" in n for n in names), names
