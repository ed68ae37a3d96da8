"""CPU oracle for paged-KV decode attention, the paged KV append and the QKV-to-cache step (f64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``paged_kv_decode_04_amd``) never imports it, and this package imports
nothing from the product path: the two share no code.  Only the seeded input generators
(``paged_kv_decode_04_amd.workloads``, which hold none of the method's arithmetic) serve both.

The arithmetic lives in ``pkv_oracle.c`` (plain C, binary64, fp16 decoded exactly); this module only marshals
numpy arrays into it.  Definitions and citations are in that file's header.  Every function here is pinned by
``tests/test_oracle.py`` against closed forms, hand-derived fixtures under ``tests/golden/``, a contiguous
brute force, and a library routine (torch's CPU ``scaled_dot_product_attention`` in float64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_pkv.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile pkv_oracle.c with gcc (IEEE semantics: no fast-math) into liboracle_pkv.so."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = f64
        lib.oracle_f16_array_to_f64.argtypes = [P, i64, P]
        lib.oracle_f16_array_to_f64.restype = None
        lib.oracle_k_index.argtypes = [i32, i32, i32, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_k_index.restype = i64
        lib.oracle_v_index.argtypes = [i32, i32, i32, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_v_index.restype = i64
        geom = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f64]
        lib.oracle_decode_attention.argtypes = geom + [P, i64, P, i32]
        lib.oracle_decode_attention.restype = ctypes.c_int
        lib.oracle_attention_weights.argtypes = geom + [i32, i32, P, P]
        lib.oracle_attention_weights.restype = ctypes.c_int
        lib.oracle_split_count.argtypes = [i32, i32, i32, i32]
        lib.oracle_split_count.restype = ctypes.c_int
        lib.oracle_split_partials.argtypes = geom + [i32, i32, P, P, P]
        lib.oracle_split_partials.restype = ctypes.c_int
        lib.oracle_split_combine.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, P]
        lib.oracle_split_combine.restype = ctypes.c_int
        lib.oracle_paged_kv_append.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P]
        lib.oracle_paged_kv_append.restype = i64
        lib.oracle_varlen_attention.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, f64,
                                                P, i64, P, i32]
        lib.oracle_varlen_attention.restype = ctypes.c_int
        lib.oracle_decode_attention_window.argtypes = geom + [i32, P, i64, P, i32]
        lib.oracle_decode_attention_window.restype = ctypes.c_int
        lib.oracle_qkv_norm_rope_paged.argtypes = [P, P, P, P, P, i32, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                                   i32, f64, i32, P, P, P, P]
        lib.oracle_qkv_norm_rope_paged.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _bits(a: np.ndarray) -> np.ndarray:
    """fp16 array -> contiguous uint16 view of its bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype == np.uint16:
        return a
    raise TypeError("expected float16 or uint16 bits, got %s" % a.dtype)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact binary16 -> binary64 decode of an array of fp16 values or bit patterns."""
    b = _bits(np.asarray(bits))
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_f16_array_to_f64(_ptr(b), b.size, _ptr(out))
    return out


def k_index(num_kv_heads, block_size, head_dim, block, head, offset, dim) -> int:
    """Flat index of K element (block, kv head, row offset, dim) in k_pool[N][Hkv][BS/16][D/32][16][32]."""
    return _load().oracle_k_index(num_kv_heads, block_size, head_dim, block, head, offset, dim)


def v_index(num_kv_heads, block_size, head_dim, block, head, offset, dim) -> int:
    """Flat index of V element (block, kv head, row offset, dim) in v_pool[N][Hkv][BS/16][4][D][4]."""
    return _load().oracle_v_index(num_kv_heads, block_size, head_dim, block, head, offset, dim)


def _geometry(q, k_pool, v_pool, block_tables, context_lens):
    B, Hq, D = q.shape
    N, Hkv, NP, D32, sixteen, w32 = k_pool.shape
    BS = NP * 16
    if (sixteen, w32) != (16, 32) or D32 * 32 != D or v_pool.shape != (N, Hkv, NP, 4, D, 4):
        raise ValueError("pool shapes %s / %s do not match q %s" % (k_pool.shape, v_pool.shape, q.shape))
    bt = _i32(block_tables)
    if bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("block_tables must be [B][M]")
    cl = _i32(context_lens)
    if cl.shape != (B,):
        raise ValueError("context_lens must be [B]")
    return B, Hq, Hkv, D, BS, N, bt.shape[1], bt, cl


def decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale, units=None, threads=None, window=0):
    """out[B][Hq][D] (or out[len(units)][D] for a list of (s, hq) units) in float64.

    q: [B][Hq][D] fp16; k_pool: [N][Hkv][BS/16][D/32][16][32] fp16; v_pool: [N][Hkv][BS/16][4][D][4] fp16;
    block_tables: [B][M] int32; context_lens: [B] int32 (rows including the newest token).
    window > 0: each new row attends only its sequence's last `window` rows (sliding-window decode).
    """
    B, Hq, Hkv, D, BS, N, M, bt, cl = _geometry(q, k_pool, v_pool, block_tables, context_lens)
    qb, kb, vb = _bits(q), _bits(k_pool), _bits(v_pool)
    if threads is None:
        threads = os.cpu_count() or 1
    if units is None:
        out = np.empty((B, Hq, D), dtype=np.float64)
        up, n = None, 0
    else:
        u = _i32(units).reshape(-1, 2)
        out = np.empty((u.shape[0], D), dtype=np.float64)
        up, n = _ptr(u), u.shape[0]
    if window:
        rc = _load().oracle_decode_attention_window(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(bt), _ptr(cl), B, Hq, Hkv, D,
                                                    BS, N, M, float(scale), int(window), up, n, _ptr(out),
                                                    int(threads))
    else:
        rc = _load().oracle_decode_attention(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(bt), _ptr(cl), B, Hq, Hkv, D, BS,
                                             N, M, float(scale), up, n, _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("oracle_decode_attention failed (%d): bad geometry or a table entry outside the pool" % rc)
    return out


def attention_weights(q, k_pool, v_pool, block_tables, context_lens, scale, s, hq):
    """(out[D], weights[L]) for one (sequence, query head): the normalised softmax weights over its rows."""
    B, Hq, Hkv, D, BS, N, M, bt, cl = _geometry(q, k_pool, v_pool, block_tables, context_lens)
    qb, kb, vb = _bits(q), _bits(k_pool), _bits(v_pool)
    L = max(int(cl[s]), 0)
    out = np.empty(D, dtype=np.float64)
    w = np.empty(max(L, 1), dtype=np.float64)
    rc = _load().oracle_attention_weights(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(bt), _ptr(cl), B, Hq, Hkv, D, BS, N,
                                          M, float(scale), int(s), int(hq), _ptr(out), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_attention_weights failed (%d)" % rc)
    return out, w[:L]


def split_count(context_len, block_size, num_splits, chunk_blocks=0) -> int:
    """Number of non-empty splits of a sequence: ceil(nb / chunk), nb = ceil(L / BS)."""
    return _load().oracle_split_count(int(context_len), int(block_size), int(num_splits), int(chunk_blocks))


def split_partials(q, k_pool, v_pool, block_tables, context_lens, scale, num_splits, chunk_blocks=0):
    """(O[B][Hq][S][D], m[B][Hq][S], l[B][Hq][S]) in float64; m in the natural-log units of z = scale*q.k."""
    B, Hq, Hkv, D, BS, N, M, bt, cl = _geometry(q, k_pool, v_pool, block_tables, context_lens)
    qb, kb, vb = _bits(q), _bits(k_pool), _bits(v_pool)
    S = int(num_splits)
    O = np.empty((B, Hq, S, D), dtype=np.float64)
    m = np.empty((B, Hq, S), dtype=np.float64)
    l = np.empty((B, Hq, S), dtype=np.float64)
    rc = _load().oracle_split_partials(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(bt), _ptr(cl), B, Hq, Hkv, D, BS, N, M,
                                       float(scale), S, int(chunk_blocks), _ptr(O), _ptr(m), _ptr(l))
    if rc != 0:
        raise ValueError("oracle_split_partials failed (%d)" % rc)
    return O, m, l


def split_combine(O, m, l, context_lens, block_size, chunk_blocks=0):
    """out[B][Hq][D] (float64) from split partials; entries of splits past ceil(nb/chunk) are never read."""
    O = np.ascontiguousarray(O, dtype=np.float64)
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    B, Hq, S, D = O.shape
    cl = _i32(context_lens)
    out = np.empty((B, Hq, D), dtype=np.float64)
    rc = _load().oracle_split_combine(_ptr(O), _ptr(m), _ptr(l), _ptr(cl), B, Hq, D, int(block_size), S,
                                      int(chunk_blocks), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_split_combine failed (%d)" % rc)
    return out


def paged_kv_append(k, v, slot_mapping, k_pool, v_pool) -> int:
    """In-place append of k, v ([T][Hkv][D] fp16) into the pools; returns the number of skipped slots."""
    kb, vb = _bits(k), _bits(v)
    T, Hkv, D = kb.shape
    N, Hkv2, NP, D32, sixteen, w32 = k_pool.shape
    BS = NP * 16
    if (Hkv2, D32 * 32, sixteen, w32) != (Hkv, D, 16, 32) or v_pool.shape != (N, Hkv, NP, 4, D, 4):
        raise ValueError("pool shapes do not match k/v")
    if not (k_pool.flags.c_contiguous and v_pool.flags.c_contiguous):
        raise ValueError("pools must be C-contiguous (updated in place)")
    sm = _i32(slot_mapping)
    if sm.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    kp = k_pool.view(np.uint16)
    vp = v_pool.view(np.uint16)
    n = _load().oracle_paged_kv_append(_ptr(kb), _ptr(vb), _ptr(sm), T, Hkv, D, BS, N, _ptr(kp), _ptr(vp))
    if n < 0:
        raise ValueError("oracle_paged_kv_append failed")
    return int(n)


def varlen_attention(q, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, scale, units=None, threads=None):
    """Paged varlen attention in float64: out[T][Hq][D] (or out[len(units)][D] for (token, hq) pairs).

    q: [T][Hq][D] fp16, token-major; sequence s owns tokens cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1, its i-th token
    at position pos_offsets[s] + i attends rows 0 .. pos_offsets[s] + i.  Pools and block_tables as decode_attention.
    """
    T, Hq, D = q.shape
    N, Hkv, NP, D32, sixteen, w32 = k_pool.shape
    BS = NP * 16
    if (sixteen, w32) != (16, 32) or D32 * 32 != D or v_pool.shape != (N, Hkv, NP, 4, D, 4):
        raise ValueError("pool shapes %s / %s do not match q %s" % (k_pool.shape, v_pool.shape, q.shape))
    bt = _i32(block_tables)
    cu = _i32(cu_seqlens_q)
    pos = _i32(pos_offsets)
    B = pos.shape[0]
    if bt.ndim != 2 or bt.shape[0] != B or cu.shape != (B + 1,):
        raise ValueError("block_tables must be [B][M], cu_seqlens_q [B+1], pos_offsets [B]")
    M = bt.shape[1]
    qb, kb, vb = _bits(q), _bits(k_pool), _bits(v_pool)
    if threads is None:
        threads = os.cpu_count() or 1
    if units is None:
        out = np.empty((T, Hq, D), dtype=np.float64)
        up, n = None, 0
    else:
        u = _i32(units).reshape(-1, 2)
        out = np.empty((u.shape[0], D), dtype=np.float64)
        up, n = _ptr(u), u.shape[0]
    rc = _load().oracle_varlen_attention(_ptr(qb), _ptr(kb), _ptr(vb), _ptr(bt), _ptr(cu), _ptr(pos), B, T, Hq, Hkv,
                                         D, BS, N, M, float(scale), up, n, _ptr(out), int(threads))
    if rc != 0:
        raise ValueError("oracle_varlen_attention failed (%d): bad geometry, prefix sums or positions, or a table "
                         "entry outside the pool" % rc)
    return out


def qkv_norm_rope_paged(qkv, q_norm_w, k_norm_w, cos, sin, cu_seqlens_q, rope_pos, cache_pos, block_tables,
                        k_pool, v_pool, eps, qk_mode):
    """Split QKV, q/k RMSNorm (qk_mode 1) or none (0), RoPE, and the paged-cache write, in float64.

    qkv: [T][(Hq + 2*Hkv)*D] fp16; q_norm_w, k_norm_w: [D] fp16 (ignored when qk_mode == 0, may be None);
    cos, sin: [P][D/2] float32 tables; sequence s owns tokens cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1, its i-th at
    RoPE position rope_pos[s] + i and cache row cache_pos[s] + i; eps is taken as a float32 (as the step receives
    it).  k_pool gives the geometry only (its piece axis is D // 32, empty for D < 32); v_pool
    (C-contiguous fp16) receives the value rows in place.  Returns (q_out [T][Hq][D] f64, k_rows [T][Hkv][D] f64,
    slots [T] int64 = block * BS + offset of each token's cache row).
    """
    qb = _bits(qkv)
    T, width = qb.shape
    N, Hkv, NP, four, D, four2 = v_pool.shape
    BS = NP * 16
    if (four, four2) != (4, 4) or k_pool.shape != (N, Hkv, NP, D // 32, 16, 32) or width % D:
        raise ValueError("pool shapes %s / %s do not match qkv %s" % (k_pool.shape, v_pool.shape, qb.shape))
    Hq = width // D - 2 * Hkv
    if Hq <= 0:
        raise ValueError("qkv rows hold no query heads")
    if not v_pool.flags.c_contiguous:
        raise ValueError("v_pool must be C-contiguous (updated in place)")
    cos = np.ascontiguousarray(cos, dtype=np.float32)
    sin = np.ascontiguousarray(sin, dtype=np.float32)
    if cos.ndim != 2 or cos.shape[1] != D // 2 or sin.shape != cos.shape:
        raise ValueError("cos and sin must be [P][D/2] float32")
    zeros = np.zeros(D, dtype=np.float16)
    qw = _bits(zeros if q_norm_w is None else np.asarray(q_norm_w, dtype=np.float16).reshape(D))
    kw = _bits(zeros if k_norm_w is None else np.asarray(k_norm_w, dtype=np.float16).reshape(D))
    bt = _i32(block_tables)
    cu, rp, cp = _i32(cu_seqlens_q), _i32(rope_pos), _i32(cache_pos)
    B = rp.shape[0]
    if bt.ndim != 2 or bt.shape[0] != B or cu.shape != (B + 1,) or cp.shape != (B,):
        raise ValueError("block_tables must be [B][M], cu_seqlens_q [B+1], rope_pos and cache_pos [B]")
    q_out = np.empty((T, Hq, D), dtype=np.float64)
    k_out = np.empty((T, Hkv, D), dtype=np.float64)
    slots = np.empty(T, dtype=np.int64)
    rc = _load().oracle_qkv_norm_rope_paged(_ptr(qb), _ptr(qw), _ptr(kw), _ptr(cos), _ptr(sin), cos.shape[0],
                                            _ptr(cu), _ptr(rp), _ptr(cp), _ptr(bt), B, T, Hq, Hkv, D, BS, N,
                                            bt.shape[1], float(np.float32(eps)), int(qk_mode), _ptr(q_out), _ptr(k_out),
                                            _ptr(slots), _ptr(v_pool.view(np.uint16)))
    if rc != 0:
        raise ValueError("oracle_qkv_norm_rope_paged failed (%d): bad geometry or mode, prefix sums, a position "
                         "outside the tables, a row past the table capacity, or a table entry outside the pool"
                         % rc)
    return q_out, k_out, slots
