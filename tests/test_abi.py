"""The C-ABI library without a GPU: it loads, exports every symbol include/pkv.h declares, the dispatcher is a pure
host function, and argument errors are reported before anything touches a device."""
import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_decode_04_amd import pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


def test_header_declares_the_binding_list():
    assert _declared() == sorted(pkv.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = pkv.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], stdout=subprocess.PIPE, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)", out))
    assert set(_declared()) <= exported
    # nothing else: the library is built with hidden visibility
    others = [l for l in out.splitlines() if " T " in l and not re.search(r"\bT pkv_", l)]
    assert not others, others[:5]


def test_library_has_gfx950_code_object():
    # the offload bundle of a library built here names its target id (amdgcn-amd-amdhsa--gfx950)
    data = open(pkv.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_version_and_empty_error():
    assert "gfx950" in pkv.version()
    assert isinstance(pkv.last_error(), str)


def _plan(**kw):
    args = dict(num_seqs=32, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, max_blocks_per_seq=128,
                max_context_hint=0, num_splits=0, cu_count=256)
    args.update(kw)
    return pkv.plan_decode(**args)


def test_dispatcher_forced_modes():
    p = _plan(num_splits=1)
    assert p["num_splits"] == 1 and p["workspace_bytes"] == 0
    p = _plan(num_splits=8)
    assert p["num_splits"] == 8 and p["chunk_blocks"] == 0
    assert p["workspace_bytes"] == pkv.decode_workspace_bytes(32, 32, 128, 8)
    assert p["workspace_bytes"] >= 32 * 32 * 8 * (128 + 2) * 4


def test_dispatcher_auto_is_a_function_of_shape_and_cu_count():
    # long contexts on few tiles split; plenty of short tiles stay single pass
    assert _plan(num_seqs=4, max_blocks_per_seq=2048)["num_splits"] > 1
    assert _plan(num_seqs=128, num_q_heads=16, num_kv_heads=16, head_dim=256, block_size=32,
                 max_blocks_per_seq=128)["num_splits"] == 1
    assert _plan(num_seqs=1, num_q_heads=4, num_kv_heads=2, head_dim=64, max_blocks_per_seq=3)["num_splits"] == 1
    # a bigger chip wants at least as many splits
    small = _plan(num_seqs=4, max_blocks_per_seq=2048, cu_count=64)["num_splits"]
    big = _plan(num_seqs=4, max_blocks_per_seq=2048, cu_count=256)["num_splits"]
    assert big >= small
    # the hint shrinks the assumed context
    assert _plan(num_seqs=4, max_blocks_per_seq=2048, max_context_hint=64)["num_splits"] <= \
        _plan(num_seqs=4, max_blocks_per_seq=2048)["num_splits"]
    # measured choices on 256 CUs: as many tiles as CUs or more run a single pass with 8 waves (head_dim <= 128)
    assert _plan(num_seqs=32, max_blocks_per_seq=128) == dict(num_splits=1, chunk_blocks=0, waves_per_group=8,
                                                              workspace_bytes=0)
    assert _plan(num_seqs=256, num_q_heads=64, max_blocks_per_seq=1024)["num_splits"] == 1
    # few long tiles split into about CUs / tiles ranges
    p = _plan(num_seqs=4, max_blocks_per_seq=2048)
    assert (p["num_splits"], p["waves_per_group"]) == (8, 8)
    # head_dim 256 keeps at most 4 waves
    assert _plan(num_seqs=128, num_q_heads=16, num_kv_heads=16, head_dim=256, block_size=32,
                 max_blocks_per_seq=128)["waves_per_group"] <= 4
    for kw in [dict(), dict(num_seqs=256, num_q_heads=64, max_blocks_per_seq=1024), dict(num_seqs=1)]:
        p = _plan(**kw)
        assert 1 <= p["num_splits"] <= 64
        assert p["waves_per_group"] in (1, 2, 4, 8)


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=30), pkv.PKV_EINVAL),            # not a multiple of Hkv
    (dict(head_dim=96), pkv.PKV_EUNSUPPORTED),
    (dict(block_size=8), pkv.PKV_EUNSUPPORTED),
    (dict(num_q_heads=8 * 17), pkv.PKV_EUNSUPPORTED),  # G = 17
    (dict(num_splits=-1), pkv.PKV_EINVAL),
    (dict(max_blocks_per_seq=0), pkv.PKV_EINVAL),
    (dict(num_seqs=-2), pkv.PKV_EINVAL),
])
def test_dispatcher_rejects_bad_geometry(kw, code):
    with pytest.raises(pkv.PkvError) as e:
        _plan(**kw)
    assert e.value.code == code
    assert pkv.last_error()


def test_entry_points_validate_before_touching_a_device():
    lib = pkv.load()
    pool = pkv.PoolDesc(8, 128, 16, 100)
    # null pointers with work to do
    rc = lib.pkv_paged_decode_attention(None, None, None, pool, None, 128, None, 4, 32, 0.1, None, 0, 0, None)
    assert rc == pkv.PKV_EINVAL and "null" in pkv.last_error()
    rc = lib.pkv_paged_kv_append(None, None, None, 4, None, None, pool, None)
    assert rc == pkv.PKV_EINVAL
    # empty batches are a no-op, also with null pointers
    assert lib.pkv_paged_decode_attention(None, None, None, pool, None, 128, None, 0, 32, 0.1, None, 0, 0,
                                          None) == pkv.PKV_OK
    assert lib.pkv_paged_kv_append(None, None, None, 0, None, None, pool, None) == pkv.PKV_OK
    # unsupported geometry and bad arguments
    bad = pkv.PoolDesc(8, 96, 16, 100)
    assert lib.pkv_paged_decode_attention(None, None, None, bad, None, 128, None, 4, 32, 0.1, None, 0, 0,
                                          None) == pkv.PKV_EUNSUPPORTED
    assert lib.pkv_paged_decode_attention(None, None, None, pool, None, 128, None, 4, 32, float("nan"), None, 0, 0,
                                          None) == pkv.PKV_EINVAL
    assert lib.pkv_paged_kv_append(None, None, None, -1, None, None, pool, None) == pkv.PKV_EINVAL
    odd = pkv.PoolDesc(8, 100, 16, 100)
    assert lib.pkv_paged_kv_append(None, None, None, 1, None, None, odd, None) == pkv.PKV_EUNSUPPORTED
    # misaligned (non-null, never dereferenced: the check fails first)
    rc = lib.pkv_paged_decode_attention(8, 16, 16, pool, 4, 128, 4, 4, 32, 0.1, 16, 0, 0, None)
    assert rc == pkv.PKV_EINVAL and "aligned" in pkv.last_error()
    # split entry points
    assert lib.pkv_paged_decode_split_partials(None, None, None, pool, None, 128, None, 4, 32, 0.1, 0, 0, None, None,
                                               None, None) == pkv.PKV_EINVAL
    assert lib.pkv_paged_decode_split_partials(None, None, None, pool, None, 128, None, 4, 32, 0.1, 4, 8, None, None,
                                               None, None) == pkv.PKV_EINVAL  # 4 * 8 < 128 blocks
    assert lib.pkv_paged_decode_split_combine(None, None, None, None, 4, 32, 96, 16, 128, 8, 0, None,
                                              None) == pkv.PKV_EUNSUPPORTED
    assert lib.pkv_paged_decode_split_combine(None, None, None, None, 0, 32, 128, 16, 128, 8, 0, None,
                                              None) == pkv.PKV_OK


def test_varlen_step_validates_before_touching_a_device():
    lib = pkv.load()
    pool = pkv.PoolDesc(8, 128, 16, 100)
    step = lib.pkv_paged_varlen_step
    # (q, k_new, v_new, k_pool, v_pool, pool, tables, M, cu, pos, B, T, Hq, scale, out, S, max_q_len, hint, stream)
    rc = step(16, None, 16, 16, 16, pool, 4, 128, 4, 4, 4, 8, 32, 0.1, 16, 0, 2, 0, None)
    assert rc == pkv.PKV_EINVAL and "k_new" in pkv.last_error()
    rc = step(16, 16, 8, 16, 16, pool, 4, 128, 4, 4, 4, 8, 32, 0.1, 16, 0, 2, 0, None)
    assert rc == pkv.PKV_EINVAL and "aligned" in pkv.last_error()
    rc = step(16, 16, 16, 16, 16, pool, 4, 128, 4, 4, 4, 8, 32, 0.1, 16, 0, 0, 0, None)  # max_q_len is required
    assert rc == pkv.PKV_EINVAL and "max_q_len" in pkv.last_error()
    assert step(None, None, None, None, None, pool, None, 128, None, None, 0, 0, 32, 0.1, None, 0, 0, 0,
                None) == pkv.PKV_OK  # empty batch
    assert step(16, 16, 16, 16, 16, pkv.PoolDesc(8, 96, 16, 100), 4, 128, 4, 4, 4, 8, 32, 0.1, 16, 0, 2, 0,
                None) == pkv.PKV_EUNSUPPORTED


def test_window_step_validates_before_touching_a_device():
    lib = pkv.load()
    pool = pkv.PoolDesc(8, 128, 16, 100)
    step = lib.pkv_paged_decode_step_window
    # (q, k_new, v_new, k_pool, v_pool, pool, tables, M, lens, B, Hq, scale, out, S, window, hint, stream)
    rc = step(16, None, 16, 16, 16, pool, 4, 128, 4, 4, 32, 0.1, 16, 0, 64, 0, None)
    assert rc == pkv.PKV_EINVAL and "k_new" in pkv.last_error()
    rc = step(16, 16, 16, 16, 16, pool, 4, 128, 4, 4, 32, 0.1, 16, 0, -1, 0, None)
    assert rc == pkv.PKV_EINVAL and "window" in pkv.last_error()
    assert step(None, None, None, None, None, pool, None, 128, None, 0, 32, 0.1, None, 0, 64, 0, None) == pkv.PKV_OK


def test_qkv_entry_points_validate_before_touching_a_device():
    lib = pkv.load()
    pool = pkv.PoolDesc(8, 128, 16, 100)
    varlen = lib.pkv_split_qkv_norm_rope_into_paged_cache_varlen
    one = lib.pkv_split_qkv_norm_rope_into_paged_cache
    # qkv, qn, kn, cos, sin, P, q_out, kp, vp, pool, bt, M, cu, pos, B, T, Hq, eps, mode, stream
    assert varlen(None, None, None, None, None, 64, None, None, None, pool, None, 128, None, None, 4, 8, 32, 1e-6, 1,
                  None) == pkv.PKV_EINVAL
    assert varlen(None, None, None, None, None, 64, None, None, None, pool, None, 128, None, None, 0, 8, 32, 1e-6, 1,
                  None) == pkv.PKV_OK  # no sequences: a no-op
    assert varlen(None, None, None, None, None, 64, None, None, None, pool, None, 128, None, None, 4, 8, 32, 1e-6, 2,
                  None) == pkv.PKV_EINVAL and "qk_mode" in pkv.last_error()
    assert varlen(None, None, None, None, None, 64, None, None, None, pool, None, 128, None, None, 4, 8, 32, -1.0, 1,
                  None) == pkv.PKV_EINVAL
    assert varlen(None, None, None, None, None, 0, None, None, None, pool, None, 128, None, None, 4, 8, 32, 1e-6, 1,
                  None) == pkv.PKV_EINVAL
    assert varlen(None, None, None, None, None, 64, None, None, None, pkv.PoolDesc(8, 96, 16, 100), None, 128, None,
                  None, 4, 8, 32, 1e-6, 1, None) == pkv.PKV_EUNSUPPORTED
    assert varlen(None, None, None, None, None, 64, None, None, None, pool, None, 128, None, None, 4, 8, 30, 1e-6, 1,
                  None) == pkv.PKV_EINVAL  # 30 query heads over 8 kv heads
    # qkv, qn, kn, cos, sin, P, q_out, kp, vp, pool, bt, M, T, Hq, pos_offset, cache_len, eps, mode, stream
    assert one(None, None, None, None, None, 64, None, None, None, pool, None, 4, 8, 32, 60, 0, 1e-6, 0,
               None) == pkv.PKV_EINVAL and "table rows" in pkv.last_error()  # positions 60..67 of 64
    assert one(None, None, None, None, None, 64, None, None, None, pool, None, 4, 8, 32, 0, 60, 1e-6, 0,
               None) == pkv.PKV_EINVAL and "capacity" in pkv.last_error()  # rows 60..67 of 4 * 16
    assert one(None, None, None, None, None, 64, None, None, None, pool, None, 4, 0, 32, 0, 0, 1e-6, 0,
               None) == pkv.PKV_OK
    # misaligned (non-null, never dereferenced)
    rc = one(8, 16, 16, 16, 16, 64, 16, 16, 16, pool, 4, 4, 8, 32, 0, 0, 1e-6, 1, None)
    assert rc == pkv.PKV_EINVAL and "aligned" in pkv.last_error()
    step = lib.pkv_paged_decode_step_qkv
    # qkv, qn, kn, cos, sin, P, eps, mode, q_out, kp, vp, pool, bt, M, cl, B, Hq, scale, out, S, hint, stream
    assert step(None, None, None, None, None, 64, 1e-6, 1, None, None, None, pool, None, 128, None, 4, 32, 0.1, None,
                0, 0, None) == pkv.PKV_EINVAL and "null" in pkv.last_error()
    assert step(None, None, None, None, None, 64, 1e-6, 3, None, None, None, pool, None, 128, None, 4, 32, 0.1, None,
                0, 0, None) == pkv.PKV_EINVAL and "qk_mode" in pkv.last_error()
    assert step(None, None, None, None, None, 0, 1e-6, 1, None, None, None, pool, None, 128, None, 4, 32, 0.1, None,
                0, 0, None) == pkv.PKV_EINVAL
    assert step(None, None, None, None, None, 64, 1e-6, 1, None, None, None, pool, None, 128, None, 0, 32, 0.1, None,
                0, 0, None) == pkv.PKV_OK  # no sequences
    assert step(None, None, None, None, None, 64, 1e-6, 1, None, None, None, pkv.PoolDesc(8, 96, 16, 100), None, 128,
                None, 4, 32, 0.1, None, 0, 0, None) == pkv.PKV_EUNSUPPORTED


def test_check_entry_points_validate_arguments():
    lib = pkv.load()
    pool = pkv.PoolDesc(8, 128, 16, 100)
    assert lib.pkv_check_decode_inputs(None, 128, None, 4, pool, 0, None, None) == pkv.PKV_EINVAL  # no report
    assert lib.pkv_check_decode_inputs(None, 128, None, 4, pool, 0, 64, None) == pkv.PKV_EINVAL  # null arrays
    assert lib.pkv_check_decode_inputs(4, 128, 4, 4, pool, -1, 64, None) == pkv.PKV_EINVAL  # negative window
    assert lib.pkv_check_decode_inputs(4, 128, 4, 4, pkv.PoolDesc(8, 128, 24, 100), 0, 64,
                                       None) == pkv.PKV_EUNSUPPORTED
    assert lib.pkv_check_varlen_inputs(None, 128, None, None, 4, 8, pool, 64, None) == pkv.PKV_EINVAL
    assert lib.pkv_check_varlen_inputs(4, 128, 4, 4, 4, -1, pool, 64, None) == pkv.PKV_EINVAL
    assert lib.pkv_check_slot_mapping(None, 3, pool, 64, None) == pkv.PKV_EINVAL
    assert lib.pkv_check_slot_mapping(None, -1, pool, 64, None) == pkv.PKV_EINVAL
    assert lib.pkv_check_slot_mapping(2, 3, pool, 64, None) == pkv.PKV_EINVAL  # misaligned


def test_workspace_bytes_layout():
    assert pkv.decode_workspace_bytes(4, 32, 128, 1) == 0
    n = pkv.decode_workspace_bytes(4, 32, 128, 16)
    o = 4 * 32 * 16 * 128 * 4
    ml = 4 * 32 * 16 * 4
    r = lambda x: (x + 255) // 256 * 256
    assert n == r(o) + 2 * r(ml)


def test_binding_without_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(pkv, "_lib", None)
    with pytest.raises(pkv.PkvError):
        pkv.load(str(tmp_path / "missing.so"))


def test_probe_library_exports_the_probe_and_rejects_bad_arguments():
    """libpkvprobe.so (the stream-read floor probe beside the library) exports what include/pkv_probe.h declares and
    refuses bad arguments before launching anything (no device needed for these)."""
    path = os.path.join(ROOT, "paged_kv_decode_04_amd", "libpkvprobe.so")
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pkv_probe.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))
    assert declared == ["pkv_probe_stream_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", path], stdout=subprocess.PIPE, text=True, check=True).stdout
    assert set(re.findall(r"\bT (pkv_\w+)", out)) == set(declared)
    lib = ctypes.CDLL(path)
    f = lib.pkv_probe_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int32,
                                                                             ctypes.c_void_p]
    assert f(None, 0, None, None, None, 0, 0, None) == 0  # nothing to do
    assert f(None, 0, None, None, None, -1, 0, None) == 1  # negative count
    assert f(None, 0, None, None, None, 4, 12, None) == 1  # write size not a multiple of 16
    assert f(None, -16, None, None, None, 4, 0, None) == 1  # negative size
    assert f(None, 0, None, None, None, 4, 0, None) == 1  # null buffers
