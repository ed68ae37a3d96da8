"""Thin Python binding of libpkv (include/pkv.h): argument marshalling only.

Each function calls the C entry point of the same name (``pkv_`` prefix dropped) with the device pointers of torch
tensors and the current HIP stream; every step of the computation runs in the library's gfx950 kernels.  PyTorch
only supplies device memory and streams.  There is no fallback: if ``libpkv.so`` is missing or fails to load, every
call raises.

Tensor layouts (all C-contiguous, on the GPU):
    q, out        [num_seqs][num_q_heads][head_dim]                 float16
    k_pool        [num_blocks][num_kv_heads][block_size/16][head_dim/32][16][32]  float16
    v_pool        [num_blocks][num_kv_heads][block_size/16][4][head_dim][4]       float16
    block_tables  [num_seqs][max_blocks_per_seq]                    int32
    context_lens  [num_seqs]                                        int32
    k, v          [num_tokens][num_kv_heads][head_dim]              float16
    slot_mapping  [num_tokens]                                      int32
    qkv           [num_tokens][(num_q_heads + 2*num_kv_heads)*head_dim]  float16
    cos, sin      [max_positions][head_dim/2]                       float32
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")
_lib = None
_lock = threading.Lock()

PKV_OK = 0
PKV_EINVAL = -1
PKV_EUNSUPPORTED = -2
PKV_EWORKSPACE = -3
PKV_EHIP = -4
PKV_ENOMEM = -5

EXPORTED = [
    "pkv_paged_kv_append",
    "pkv_paged_decode_attention",
    "pkv_paged_decode_attention_ws",
    "pkv_paged_decode_attention_noalloc",
    "pkv_paged_decode_attention_planned",
    "pkv_paged_decode_step",
    "pkv_paged_decode_step_qkv",
    "pkv_paged_varlen_attention",
    "pkv_paged_varlen_step",
    "pkv_paged_decode_attention_window",
    "pkv_paged_decode_step_window",
    "pkv_split_qkv_norm_rope_into_paged_cache_varlen",
    "pkv_split_qkv_norm_rope_into_paged_cache",
    "pkv_plan_decode",
    "pkv_decode_workspace_bytes",
    "pkv_paged_decode_split_partials",
    "pkv_paged_decode_split_combine",
    "pkv_check_decode_inputs",
    "pkv_check_varlen_inputs",
    "pkv_check_slot_mapping",
    "pkv_device_cu_count",
    "pkv_last_error",
    "pkv_version",
]


class PkvError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__("libpkv error %d: %s" % (code, message))
        self.code = code


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32)]


class DecodePlan(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("chunk_blocks", ctypes.c_int32),
                ("waves_per_group", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libpkv.so (once) and declare the signatures; raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        # torch first: its HIP runtime must be the one libpkv binds to (loading libpkv first would bring in a
        # second runtime from the system ROCm that does not share torch's device state)
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(p):
            raise PkvError(PKV_EINVAL, "%s is not built; run __graft_entry__.build() or "
                           "python -m paged_kv_decode_04_amd.build" % p)
        lib = ctypes.CDLL(p)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        lib.pkv_paged_kv_append.argtypes = [vp, vp, vp, i32, vp, vp, PoolDesc, vp]
        attn = [vp, vp, vp, PoolDesc, vp, i32, vp, i32, i32, f32, vp, i32, i32]
        lib.pkv_paged_decode_attention.argtypes = attn + [vp]
        lib.pkv_paged_decode_attention_ws.argtypes = attn + [vp, sz, vp]
        lib.pkv_paged_decode_attention_noalloc.argtypes = attn + [vp]
        lib.pkv_paged_decode_attention_planned.argtypes = attn[:11] + [ctypes.POINTER(DecodePlan), vp, sz, vp]
        lib.pkv_paged_decode_step.argtypes = [vp, vp, vp, vp, vp, PoolDesc, vp, i32, vp, i32, i32, f32, vp, i32, i32,
                                              vp]
        lib.pkv_paged_decode_step_qkv.argtypes = [vp, vp, vp, vp, vp, i32, f32, i32, vp, vp, vp, PoolDesc, vp, i32, vp,
                                                  i32, i32, f32, vp, i32, i32, vp]
        lib.pkv_paged_decode_attention_window.argtypes = attn[:12] + [i32, i32, vp]
        lib.pkv_paged_decode_step_window.argtypes = [vp, vp, vp, vp, vp, PoolDesc, vp, i32, vp, i32, i32, f32, vp,
                                                     i32, i32, i32, vp]
        lib.pkv_paged_varlen_attention.argtypes = [vp, vp, vp, PoolDesc, vp, i32, vp, vp, i32, i32, i32, f32, vp, i32,
                                                   i32, i32, vp]
        lib.pkv_paged_varlen_step.argtypes = [vp, vp, vp, vp, vp, PoolDesc, vp, i32, vp, vp, i32, i32, i32, f32, vp,
                                              i32, i32, i32, vp]
        qkv = [vp, vp, vp, vp, vp, i32, vp, vp, vp, PoolDesc, vp, i32]
        lib.pkv_split_qkv_norm_rope_into_paged_cache_varlen.argtypes = qkv + [vp, vp, i32, i32, i32, f32, i32, vp]
        lib.pkv_split_qkv_norm_rope_into_paged_cache.argtypes = qkv + [i32, i32, i32, i32, f32, i32, vp]
        lib.pkv_plan_decode.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(DecodePlan)]
        lib.pkv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.pkv_decode_workspace_bytes.restype = sz
        lib.pkv_paged_decode_split_partials.argtypes = [vp, vp, vp, PoolDesc, vp, i32, vp, i32, i32, f32, i32, i32,
                                                        vp, vp, vp, vp]
        lib.pkv_paged_decode_split_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp]
        lib.pkv_check_decode_inputs.argtypes = [vp, i32, vp, i32, PoolDesc, i32, vp, vp]
        lib.pkv_check_varlen_inputs.argtypes = [vp, i32, vp, vp, i32, i32, PoolDesc, vp, vp]
        lib.pkv_check_slot_mapping.argtypes = [vp, i32, PoolDesc, vp, vp]
        lib.pkv_device_cu_count.argtypes = [ctypes.POINTER(i32)]
        lib.pkv_last_error.restype = ctypes.c_char_p
        lib.pkv_version.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name not in ("pkv_decode_workspace_bytes", "pkv_last_error", "pkv_version"):
                getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def _check(rc: int) -> None:
    if rc != PKV_OK:
        raise PkvError(rc, load().pkv_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t, dtype, name: str, ndim: Optional[int] = None):
    import torch
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    return t


def _pool(k_pool, v_pool) -> PoolDesc:
    import torch
    _dev(k_pool, torch.float16, "k_pool", 6)
    _dev(v_pool, torch.float16, "v_pool", 6)
    N, Hkv, NP, D32, sixteen, w32 = k_pool.shape
    D, BS = D32 * 32, NP * 16
    if (sixteen, w32) != (16, 32):
        raise ValueError("k_pool must be [N][Hkv][BS/16][D/32][16][32], got %s" % (tuple(k_pool.shape),))
    if tuple(v_pool.shape) != (N, Hkv, NP, 4, D, 4):
        raise ValueError("v_pool must be [N][Hkv][BS/16][4][D][4] = %s, got %s"
                         % ((N, Hkv, NP, 4, D, 4), tuple(v_pool.shape)))
    return PoolDesc(Hkv, D, BS, N)


def version() -> str:
    return load().pkv_version().decode()


def last_error() -> str:
    return load().pkv_last_error().decode()


def device_cu_count() -> int:
    n = ctypes.c_int32(0)
    _check(load().pkv_device_cu_count(ctypes.byref(n)))
    return n.value


def paged_kv_append(k, v, slot_mapping, k_pool, v_pool, stream=None) -> None:
    """Copy each token's K/V rows into the pools at its slot (pkv_paged_kv_append)."""
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(k, torch.float16, "k", 3)
    _dev(v, torch.float16, "v", 3)
    _dev(slot_mapping, torch.int32, "slot_mapping", 1)
    T = int(slot_mapping.shape[0])
    if tuple(k.shape) != (T, pool.num_kv_heads, pool.head_dim) or k.shape != v.shape:
        raise ValueError("k and v must be [T][Hkv][D] = %s" % ((T, pool.num_kv_heads, pool.head_dim),))
    _check(load().pkv_paged_kv_append(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_pool), _ptr(v_pool), pool,
                                      _stream(stream)))


def _attn_args(q, k_pool, v_pool, block_tables, context_lens):
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(q, torch.float16, "q", 3)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(context_lens, torch.int32, "context_lens", 1)
    B, Hq, D = q.shape
    if D != pool.head_dim:
        raise ValueError("q head_dim %d != pool head_dim %d" % (D, pool.head_dim))
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables / context_lens must have num_seqs = %d rows" % B)
    return pool, int(B), int(Hq), int(block_tables.shape[1])


def paged_decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale: float, out=None,
                           num_splits: int = 0, max_context_hint: int = 0, workspace=None, stream=None):
    """out = softmax(scale * q.K^T).V per (sequence, query head) over the paged pools.

    num_splits: 0 = dispatcher, 1 = single pass, > 1 = forced split count.  With ``workspace`` (a uint8 GPU tensor)
    the _ws entry point is called and the partials go there; otherwise the library's own workspace is used."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, torch.float16, "out", 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    lib = load()
    args = [_ptr(q), _ptr(k_pool), _ptr(v_pool), pool, _ptr(block_tables), M, _ptr(context_lens), B, Hq,
            float(scale), _ptr(out), int(num_splits), int(max_context_hint)]
    if workspace is None:
        _check(lib.pkv_paged_decode_attention(*args, _stream(stream)))
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        nbytes = workspace.numel() * workspace.element_size()
        _check(lib.pkv_paged_decode_attention_ws(*args, _ptr(workspace), nbytes, _stream(stream)))
    return out


def paged_decode_attention_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                                   num_splits: int = 0, max_context_hint: int = 0, stream=None):
    """pkv_paged_decode_attention_noalloc: decode attention whose split-K partials and dispatch-order records use the
    library's fixed device scratch (PKV_NOALLOC_SCRATCH_BYTES per device) -- the call allocates nothing, so ``out``
    must be given.  Calls on one device share that scratch: calls that may overlap in time race."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    _dev(out, torch.float16, "out", 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _check(load().pkv_paged_decode_attention_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), pool, _ptr(block_tables),
                                                     M, _ptr(context_lens), B, Hq, float(scale), _ptr(out),
                                                     int(num_splits), int(max_context_hint), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 16 << 20  # PKV_NOALLOC_SCRATCH_BYTES in include/pkv.h


def paged_decode_attention_planned(q, k_pool, v_pool, block_tables, context_lens, scale: float, plan: dict,
                                   out=None, workspace=None, stream=None):
    """Decode attention with an explicit launch plan (pkv_paged_decode_attention_planned); ``plan`` has the keys
    num_splits, chunk_blocks, waves_per_group.  workspace=None uses the library's own."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out", 3)
    pl = DecodePlan(int(plan["num_splits"]), int(plan.get("chunk_blocks", 0)), int(plan["waves_per_group"]), 0, 0)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().pkv_paged_decode_attention_planned(_ptr(q), _ptr(k_pool), _ptr(v_pool), pool, _ptr(block_tables),
                                                     M, _ptr(context_lens), B, Hq, float(scale), _ptr(out),
                                                     ctypes.byref(pl), _ptr(workspace), nbytes, _stream(stream)))
    return out


def paged_decode_step(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale: float, out=None,
                      num_splits: int = 0, max_context_hint: int = 0, stream=None):
    """Fused decode step (pkv_paged_decode_step): write each sequence's new K/V row at position L-1, then attend."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    _dev(k_new, torch.float16, "k_new", 3)
    _dev(v_new, torch.float16, "v_new", 3)
    if tuple(k_new.shape) != (B, pool.num_kv_heads, pool.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be [B][Hkv][D] = %s" % ((B, pool.num_kv_heads, pool.head_dim),))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out", 3)
    _check(load().pkv_paged_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), pool,
                                        _ptr(block_tables), M, _ptr(context_lens), B, Hq, float(scale), _ptr(out),
                                        int(num_splits), int(max_context_hint), _stream(stream)))
    return out


def paged_decode_step_window(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale: float, window: int,
                             out=None, num_splits: int = 0, max_context_hint: int = 0, stream=None):
    """Decode step with a sliding window (pkv_paged_decode_step_window): write each sequence's new K/V row at
    position L-1, then attend its last `window` rows."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    _dev(k_new, torch.float16, "k_new", 3)
    _dev(v_new, torch.float16, "v_new", 3)
    if tuple(k_new.shape) != (B, pool.num_kv_heads, pool.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be [B][Hkv][D] = %s" % ((B, pool.num_kv_heads, pool.head_dim),))
    if out is None:
        out = torch.empty_like(q)
    _dev(out, torch.float16, "out", 3)
    _check(load().pkv_paged_decode_step_window(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), pool,
                                               _ptr(block_tables), M, _ptr(context_lens), B, Hq, float(scale),
                                               _ptr(out), int(num_splits), int(window), int(max_context_hint),
                                               _stream(stream)))
    return out


def prepare_decode_step_window(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale: float,
                               window: int, out, num_splits: int = 0, max_context_hint: int = 0,
                               stream=None) -> "PreparedCall":
    """pkv_paged_decode_step_window with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, torch.float16, n, 3)
        if tuple(t.shape) != (B, pool.num_kv_heads, pool.head_dim):
            raise ValueError("%s must be [B][Hkv][D]" % n)
    _dev(out, torch.float16, "out", 3)
    lib = load()
    args = (ctypes.c_void_p(_ptr(q)), ctypes.c_void_p(_ptr(k_new)), ctypes.c_void_p(_ptr(v_new)),
            ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool, ctypes.c_void_p(_ptr(block_tables)),
            ctypes.c_int32(M), ctypes.c_void_p(_ptr(context_lens)), ctypes.c_int32(B), ctypes.c_int32(Hq),
            ctypes.c_float(scale), ctypes.c_void_p(_ptr(out)), ctypes.c_int32(num_splits), ctypes.c_int32(window),
            ctypes.c_int32(max_context_hint), ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_decode_step_window, args, (q, k_new, v_new, k_pool, v_pool, block_tables,
                                                                 context_lens, out))


def _step_qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool, block_tables, context_lens, num_q_heads,
                   qk_mode, q_out):
    import torch
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(context_lens, torch.int32, "context_lens", 1)
    pool, T, P = _qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, q_out, k_pool, v_pool, num_q_heads, qk_mode)
    B = int(context_lens.shape[0])
    if T != B or block_tables.shape[0] != B:
        raise ValueError("qkv, block_tables and context_lens must have num_seqs = %d rows" % B)
    return pool, B, P


def paged_decode_step_qkv(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool, block_tables, context_lens,
                          num_q_heads: int, scale: float, eps: float, qk_mode: int = 1, q_out=None, out=None,
                          num_splits: int = 0, max_context_hint: int = 0, stream=None):
    """Decode step from the QKV projection rows (pkv_paged_decode_step_qkv): RMS norm (qk_mode 1) and RoPE of each
    sequence's new token at position L-1, its K/V rows written to row L-1, then decode attention.  Returns
    (out, q_out)."""
    import torch
    B, D = int(context_lens.shape[0]), v_pool.shape[4]
    if q_out is None:
        q_out = torch.empty((B, int(num_q_heads), D), dtype=torch.float16, device=qkv.device)
    if out is None:
        out = torch.empty_like(q_out)
    _dev(out, torch.float16, "out", 3)
    pool, B, P = _step_qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool, block_tables, context_lens,
                                num_q_heads, qk_mode, q_out)
    _check(load().pkv_paged_decode_step_qkv(
        _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(cos), _ptr(sin), P, float(eps), int(qk_mode), _ptr(q_out),
        _ptr(k_pool), _ptr(v_pool), pool, _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), B,
        int(num_q_heads), float(scale), _ptr(out), int(num_splits), int(max_context_hint), _stream(stream)))
    return out, q_out


def plan_decode(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                max_blocks_per_seq: int, max_context_hint: int = 0, num_splits: int = 0, cu_count: int = 0) -> dict:
    """The dispatcher's plan (pkv_plan_decode); cu_count > 0 keeps it a pure host computation."""
    plan = DecodePlan()
    _check(load().pkv_plan_decode(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                  max_context_hint, num_splits, cu_count, ctypes.byref(plan)))
    return {"num_splits": plan.num_splits, "chunk_blocks": plan.chunk_blocks,
            "waves_per_group": plan.waves_per_group, "workspace_bytes": int(plan.workspace_bytes)}


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, num_splits: int) -> int:
    return int(load().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, num_splits))


def paged_decode_split_partials(q, k_pool, v_pool, block_tables, context_lens, scale: float, num_splits: int,
                                chunk_blocks: int, partial_out, partial_m, partial_l, stream=None) -> None:
    """Split-K phase 1 (pkv_paged_decode_split_partials) into caller float32 buffers
    partial_out [B][Hq][S][D], partial_m / partial_l [B][Hq][S]."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    S = int(num_splits)
    _dev(partial_out, torch.float32, "partial_out", 4)
    _dev(partial_m, torch.float32, "partial_m", 3)
    _dev(partial_l, torch.float32, "partial_l", 3)
    if tuple(partial_out.shape) != (B, Hq, S, pool.head_dim) or tuple(partial_m.shape) != (B, Hq, S) \
            or tuple(partial_l.shape) != (B, Hq, S):
        raise ValueError("partial buffers must be [B][Hq][S][D] and [B][Hq][S]")
    _check(load().pkv_paged_decode_split_partials(_ptr(q), _ptr(k_pool), _ptr(v_pool), pool, _ptr(block_tables), M,
                                                  _ptr(context_lens), B, Hq, float(scale), S, int(chunk_blocks),
                                                  _ptr(partial_out), _ptr(partial_m), _ptr(partial_l),
                                                  _stream(stream)))


def paged_decode_split_combine(partial_out, partial_m, partial_l, context_lens, block_size: int,
                               max_blocks_per_seq: int, chunk_blocks: int, out=None, stream=None):
    """Split-K phase 2 (pkv_paged_decode_split_combine): log-sum-exp combine into fp16 out [B][Hq][D]."""
    import torch
    _dev(partial_out, torch.float32, "partial_out", 4)
    _dev(partial_m, torch.float32, "partial_m", 3)
    _dev(partial_l, torch.float32, "partial_l", 3)
    _dev(context_lens, torch.int32, "context_lens", 1)
    B, Hq, S, D = partial_out.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float16, device=partial_out.device)
    _dev(out, torch.float16, "out", 3)
    _check(load().pkv_paged_decode_split_combine(_ptr(partial_out), _ptr(partial_m), _ptr(partial_l),
                                                 _ptr(context_lens), int(B), int(Hq), int(D), int(block_size),
                                                 int(max_blocks_per_seq), int(S), int(chunk_blocks), _ptr(out),
                                                 _stream(stream)))
    return out


def paged_decode_attention_window(q, k_pool, v_pool, block_tables, context_lens, scale: float, window: int,
                                  out=None, num_splits: int = 0, max_context_hint: int = 0, stream=None):
    """Sliding-window decode attention (pkv_paged_decode_attention_window): each sequence's new row attends only its
    last ``window`` rows (window = 0: all rows)."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, torch.float16, "out", 3)
    _check(load().pkv_paged_decode_attention_window(_ptr(q), _ptr(k_pool), _ptr(v_pool), pool, _ptr(block_tables),
                                                    M, _ptr(context_lens), B, Hq, float(scale), _ptr(out),
                                                    int(num_splits), int(window), int(max_context_hint),
                                                    _stream(stream)))
    return out


def paged_varlen_attention(q, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, scale: float, out=None,
                           num_splits: int = 0, max_q_len: int = 0, max_context_hint: int = 0, stream=None):
    """Attention of several new query rows per sequence (pkv_paged_varlen_attention): q and out are token-major
    [T][Hq][D]; sequence s owns rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1, its i-th new row at position
    pos_offsets[s] + i attending rows 0 .. pos_offsets[s] + i.  The pools must already hold the new rows."""
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(q, torch.float16, "q", 3)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _dev(pos_offsets, torch.int32, "pos_offsets", 1)
    T, Hq, D = q.shape
    B = int(pos_offsets.shape[0])
    if D != pool.head_dim:
        raise ValueError("q head_dim %d != pool head_dim %d" % (D, pool.head_dim))
    if block_tables.shape[0] != B or cu_seqlens_q.shape[0] != B + 1:
        raise ValueError("block_tables must have num_seqs = %d rows and cu_seqlens_q num_seqs + 1 entries" % B)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, torch.float16, "out", 3)
    _check(load().pkv_paged_varlen_attention(_ptr(q), _ptr(k_pool), _ptr(v_pool), pool, _ptr(block_tables),
                                             int(block_tables.shape[1]), _ptr(cu_seqlens_q), _ptr(pos_offsets), B,
                                             int(T), int(Hq), float(scale), _ptr(out), int(num_splits),
                                             int(max_q_len), int(max_context_hint), _stream(stream)))
    return out


def _varlen_step_args(q, k_new, v_new, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets):
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(q, torch.float16, "q", 3)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _dev(pos_offsets, torch.int32, "pos_offsets", 1)
    T = int(q.shape[0])
    B = int(pos_offsets.shape[0])
    if q.shape[2] != pool.head_dim:
        raise ValueError("q head_dim %d != pool head_dim %d" % (q.shape[2], pool.head_dim))
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, torch.float16, n, 3)
        if tuple(t.shape) != (T, pool.num_kv_heads, pool.head_dim):
            raise ValueError("%s must be [T][Hkv][D] = %s" % (n, (T, pool.num_kv_heads, pool.head_dim)))
    if block_tables.shape[0] != B or cu_seqlens_q.shape[0] != B + 1:
        raise ValueError("block_tables must have num_seqs = %d rows and cu_seqlens_q num_seqs + 1 entries" % B)
    return pool, B, T


def paged_varlen_step(q, k_new, v_new, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, scale: float,
                      max_q_len: int, out=None, num_splits: int = 0, max_context_hint: int = 0, stream=None):
    """The varlen step (pkv_paged_varlen_step): token t's new K/V rows (k_new, v_new: [T][Hkv][D]) go to row
    pos_offsets[s] + i of its sequence, then every new row attends as in paged_varlen_attention.  max_q_len bounds
    every sequence's new rows (required)."""
    import torch
    pool, B, T = _varlen_step_args(q, k_new, v_new, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, torch.float16, "out", 3)
    _check(load().pkv_paged_varlen_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), pool,
                                        _ptr(block_tables), int(block_tables.shape[1]), _ptr(cu_seqlens_q),
                                        _ptr(pos_offsets), B, T, int(q.shape[1]), float(scale), _ptr(out),
                                        int(num_splits), int(max_q_len), int(max_context_hint), _stream(stream)))
    return out


def _qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, q_out, k_pool, v_pool, num_q_heads: int, qk_mode: int):
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(qkv, torch.float16, "qkv", 2)
    _dev(cos, torch.float32, "cos", 2)
    _dev(sin, torch.float32, "sin", 2)
    _dev(q_out, torch.float16, "q_out", 3)
    D, Hkv, Hq = pool.head_dim, pool.num_kv_heads, int(num_q_heads)
    T = int(qkv.shape[0])
    if qkv.shape[1] != (Hq + 2 * Hkv) * D:
        raise ValueError("qkv rows must hold (Hq + 2*Hkv) * D = %d values" % ((Hq + 2 * Hkv) * D))
    if tuple(q_out.shape) != (T, Hq, D):
        raise ValueError("q_out must be [T][Hq][D] = %s" % ((T, Hq, D),))
    if cos.shape[1] != D // 2 or cos.shape != sin.shape:
        raise ValueError("cos and sin must be [max_positions][D/2]")
    for w, n in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _dev(w, torch.float16, n, 1)
            if w.shape[0] != D:
                raise ValueError("%s must hold head_dim values" % n)
        elif qk_mode == 1:
            raise ValueError("qk_mode 1 needs %s" % n)
    return pool, T, int(cos.shape[0])


def split_qkv_norm_rope_into_paged_cache_varlen(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool, block_tables,
                                                cu_seqlens_q, pos_offsets, num_q_heads: int, eps: float,
                                                qk_mode: int = 1, q_out=None, stream=None):
    """The step before attention (pkv_split_qkv_norm_rope_into_paged_cache_varlen): from qkv [T][(Hq+2Hkv)*D],
    RMS-normalise (qk_mode 1) and rotate the query and key heads, write q_out [T][Hq][D] and each token's K/V rows
    into the pools at row pos_offsets[s] + i of its sequence.  Returns q_out."""
    import torch
    if q_out is None:
        q_out = torch.empty((qkv.shape[0], int(num_q_heads), v_pool.shape[4]), dtype=torch.float16,
                            device=qkv.device)
    pool, T, P = _qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, q_out, k_pool, v_pool, num_q_heads, qk_mode)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _dev(pos_offsets, torch.int32, "pos_offsets", 1)
    B = int(pos_offsets.shape[0])
    if block_tables.shape[0] != B or cu_seqlens_q.shape[0] != B + 1:
        raise ValueError("block_tables must have num_seqs = %d rows and cu_seqlens_q num_seqs + 1 entries" % B)
    _check(load().pkv_split_qkv_norm_rope_into_paged_cache_varlen(
        _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(cos), _ptr(sin), P, _ptr(q_out), _ptr(k_pool), _ptr(v_pool),
        pool, _ptr(block_tables), int(block_tables.shape[1]), _ptr(cu_seqlens_q), _ptr(pos_offsets), B, T,
        int(num_q_heads), float(eps), int(qk_mode), _stream(stream)))
    return q_out


def split_qkv_norm_rope_into_paged_cache(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool, block_table,
                                         num_q_heads: int, pos_offset: int, cache_len: int, eps: float,
                                         qk_mode: int = 1, q_out=None, stream=None):
    """One-sequence form (pkv_split_qkv_norm_rope_into_paged_cache): token i takes RoPE position pos_offset + i and
    cache row cache_len + i of the sequence whose table is block_table [M].  Returns q_out."""
    import torch
    if q_out is None:
        q_out = torch.empty((qkv.shape[0], int(num_q_heads), v_pool.shape[4]), dtype=torch.float16,
                            device=qkv.device)
    pool, T, P = _qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, q_out, k_pool, v_pool, num_q_heads, qk_mode)
    _dev(block_table, torch.int32, "block_table", 1)
    _check(load().pkv_split_qkv_norm_rope_into_paged_cache(
        _ptr(qkv), _ptr(q_norm_w), _ptr(k_norm_w), _ptr(cos), _ptr(sin), P, _ptr(q_out), _ptr(k_pool), _ptr(v_pool),
        pool, _ptr(block_table), int(block_table.shape[0]), T, int(num_q_heads), int(pos_offset), int(cache_len),
        float(eps), int(qk_mode), _stream(stream)))
    return q_out


def _report(report, device):
    import torch
    if report is None:
        return torch.empty(4, dtype=torch.int32, device=device)
    _dev(report, torch.int32, "report", 1)
    if report.shape[0] < 4:
        raise ValueError("report must hold 4 int32")
    return report


def check_decode_inputs(k_pool, v_pool, block_tables, context_lens, window: int = 0, report=None, stream=None):
    """Device-side check of decode inputs (pkv_check_decode_inputs); returns the int32[4] report tensor (read it
    after synchronising: bad lengths, bad table entries, first bad sequence or INT32_MAX)."""
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(context_lens, torch.int32, "context_lens", 1)
    report = _report(report, block_tables.device)
    _check(load().pkv_check_decode_inputs(_ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens),
                                          int(context_lens.shape[0]), pool, int(window), _ptr(report),
                                          _stream(stream)))
    return report


def check_varlen_inputs(k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, total_q_tokens: int, report=None,
                        stream=None):
    """Device-side check of varlen inputs (pkv_check_varlen_inputs); returns the int32[4] report tensor."""
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(block_tables, torch.int32, "block_tables", 2)
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _dev(pos_offsets, torch.int32, "pos_offsets", 1)
    report = _report(report, block_tables.device)
    _check(load().pkv_check_varlen_inputs(_ptr(block_tables), int(block_tables.shape[1]), _ptr(cu_seqlens_q),
                                          _ptr(pos_offsets), int(pos_offsets.shape[0]), int(total_q_tokens), pool,
                                          _ptr(report), _stream(stream)))
    return report


def check_slot_mapping(k_pool, v_pool, slot_mapping, report=None, stream=None):
    """Device-side check of an append's slot mapping (pkv_check_slot_mapping); returns the int32[4] report."""
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(slot_mapping, torch.int32, "slot_mapping", 1)
    report = _report(report, slot_mapping.device)
    _check(load().pkv_check_slot_mapping(_ptr(slot_mapping), int(slot_mapping.shape[0]), pool, _ptr(report),
                                         _stream(stream)))
    return report


class PreparedCall:
    """A C entry point with its arguments marshalled once (device pointers, geometry, stream).  Calling it costs one
    ctypes call and no Python-side checks: for tight decode loops where per-call marshalling would outlast the
    kernel.  The tensors must stay alive, keep their storage, and the stream stay valid while the object is used."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep  # tensors referenced by the pointers

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != PKV_OK:
            _check(rc)


def prepare_decode_step(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                        num_splits: int = 0, max_context_hint: int = 0, stream=None) -> PreparedCall:
    """pkv_paged_decode_step with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _dev(t, torch.float16, n, 3)
        if tuple(t.shape) != (B, pool.num_kv_heads, pool.head_dim):
            raise ValueError("%s must be [B][Hkv][D]" % n)
    _dev(out, torch.float16, "out", 3)
    lib = load()
    args = (ctypes.c_void_p(_ptr(q)), ctypes.c_void_p(_ptr(k_new)), ctypes.c_void_p(_ptr(v_new)),
            ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool, ctypes.c_void_p(_ptr(block_tables)),
            ctypes.c_int32(M), ctypes.c_void_p(_ptr(context_lens)), ctypes.c_int32(B), ctypes.c_int32(Hq),
            ctypes.c_float(scale), ctypes.c_void_p(_ptr(out)), ctypes.c_int32(num_splits),
            ctypes.c_int32(max_context_hint), ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_decode_step, args, (q, k_new, v_new, k_pool, v_pool, block_tables,
                                                          context_lens, out))


def prepare_paged_decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                                   num_splits: int = 0, max_context_hint: int = 0, stream=None) -> PreparedCall:
    """pkv_paged_decode_attention with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    _dev(out, torch.float16, "out", 3)
    lib = load()
    args = (ctypes.c_void_p(_ptr(q)), ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool,
            ctypes.c_void_p(_ptr(block_tables)), ctypes.c_int32(M), ctypes.c_void_p(_ptr(context_lens)),
            ctypes.c_int32(B), ctypes.c_int32(Hq), ctypes.c_float(scale), ctypes.c_void_p(_ptr(out)),
            ctypes.c_int32(num_splits), ctypes.c_int32(max_context_hint), ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_decode_attention, args, (q, k_pool, v_pool, block_tables, context_lens, out))


def prepare_paged_decode_attention_planned(q, k_pool, v_pool, block_tables, context_lens, scale: float, plan: dict,
                                           out, workspace=None, stream=None) -> PreparedCall:
    """pkv_paged_decode_attention_planned with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    _dev(out, torch.float16, "out", 3)
    pl = DecodePlan(int(plan["num_splits"]), int(plan.get("chunk_blocks", 0)), int(plan["waves_per_group"]), 0, 0)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = load()
    args = (ctypes.c_void_p(_ptr(q)), ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool,
            ctypes.c_void_p(_ptr(block_tables)), ctypes.c_int32(M), ctypes.c_void_p(_ptr(context_lens)),
            ctypes.c_int32(B), ctypes.c_int32(Hq), ctypes.c_float(scale), ctypes.c_void_p(_ptr(out)),
            ctypes.byref(pl), ctypes.c_void_p(_ptr(workspace)), ctypes.c_size_t(nbytes),
            ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_decode_attention_planned, args,
                        (q, k_pool, v_pool, block_tables, context_lens, out, workspace, pl))


def prepare_paged_varlen_attention(q, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, scale: float, out,
                                   num_splits: int = 0, max_q_len: int = 0, max_context_hint: int = 0,
                                   stream=None) -> PreparedCall:
    """pkv_paged_varlen_attention with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(q, torch.float16, "q", 3)
    _dev(out, torch.float16, "out", 3)
    B = int(pos_offsets.shape[0])
    lib = load()
    args = (ctypes.c_void_p(_ptr(q)), ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool,
            ctypes.c_void_p(_ptr(block_tables)), ctypes.c_int32(int(block_tables.shape[1])),
            ctypes.c_void_p(_ptr(cu_seqlens_q)), ctypes.c_void_p(_ptr(pos_offsets)), ctypes.c_int32(B),
            ctypes.c_int32(int(q.shape[0])), ctypes.c_int32(int(q.shape[1])), ctypes.c_float(scale),
            ctypes.c_void_p(_ptr(out)), ctypes.c_int32(num_splits), ctypes.c_int32(max_q_len),
            ctypes.c_int32(max_context_hint), ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_varlen_attention, args,
                        (q, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, out))


def prepare_paged_varlen_step(q, k_new, v_new, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets,
                              scale: float, max_q_len: int, out, num_splits: int = 0, max_context_hint: int = 0,
                              stream=None) -> PreparedCall:
    """pkv_paged_varlen_step with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool, B, T = _varlen_step_args(q, k_new, v_new, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets)
    _dev(out, torch.float16, "out", 3)
    lib = load()
    args = (ctypes.c_void_p(_ptr(q)), ctypes.c_void_p(_ptr(k_new)), ctypes.c_void_p(_ptr(v_new)),
            ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool, ctypes.c_void_p(_ptr(block_tables)),
            ctypes.c_int32(int(block_tables.shape[1])), ctypes.c_void_p(_ptr(cu_seqlens_q)),
            ctypes.c_void_p(_ptr(pos_offsets)), ctypes.c_int32(B), ctypes.c_int32(T), ctypes.c_int32(int(q.shape[1])),
            ctypes.c_float(scale), ctypes.c_void_p(_ptr(out)), ctypes.c_int32(num_splits), ctypes.c_int32(max_q_len),
            ctypes.c_int32(max_context_hint), ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_varlen_step, args,
                        (q, k_new, v_new, k_pool, v_pool, block_tables, cu_seqlens_q, pos_offsets, out))


def prepare_paged_decode_attention_window(q, k_pool, v_pool, block_tables, context_lens, scale: float, out,
                                          window: int, num_splits: int = 0, max_context_hint: int = 0,
                                          stream=None) -> PreparedCall:
    """pkv_paged_decode_attention_window with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool, B, Hq, M = _attn_args(q, k_pool, v_pool, block_tables, context_lens)
    _dev(out, torch.float16, "out", 3)
    lib = load()
    args = (ctypes.c_void_p(_ptr(q)), ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool,
            ctypes.c_void_p(_ptr(block_tables)), ctypes.c_int32(M), ctypes.c_void_p(_ptr(context_lens)),
            ctypes.c_int32(B), ctypes.c_int32(Hq), ctypes.c_float(scale), ctypes.c_void_p(_ptr(out)),
            ctypes.c_int32(num_splits), ctypes.c_int32(window), ctypes.c_int32(max_context_hint),
            ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_decode_attention_window, args,
                        (q, k_pool, v_pool, block_tables, context_lens, out))


def prepare_paged_kv_append(k, v, slot_mapping, k_pool, v_pool, stream=None) -> PreparedCall:
    """pkv_paged_kv_append with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool = _pool(k_pool, v_pool)
    _dev(k, torch.float16, "k", 3)
    _dev(v, torch.float16, "v", 3)
    _dev(slot_mapping, torch.int32, "slot_mapping", 1)
    T = int(slot_mapping.shape[0])
    if tuple(k.shape) != (T, pool.num_kv_heads, pool.head_dim) or k.shape != v.shape:
        raise ValueError("k and v must be [T][Hkv][D]")
    lib = load()
    args = (ctypes.c_void_p(_ptr(k)), ctypes.c_void_p(_ptr(v)), ctypes.c_void_p(_ptr(slot_mapping)),
            ctypes.c_int32(T), ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool,
            ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_kv_append, args, (k, v, slot_mapping, k_pool, v_pool))


def prepare_split_qkv_norm_rope_into_paged_cache_varlen(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool,
                                                        block_tables, cu_seqlens_q, pos_offsets, num_q_heads: int,
                                                        eps: float, qk_mode: int, q_out,
                                                        stream=None) -> PreparedCall:
    """pkv_split_qkv_norm_rope_into_paged_cache_varlen with its arguments marshalled once (see PreparedCall)."""
    import torch
    pool, T, P = _qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, q_out, k_pool, v_pool, num_q_heads, qk_mode)
    _dev(block_tables, torch.int32, "block_tables", 2)
    B = int(pos_offsets.shape[0])
    lib = load()
    args = (ctypes.c_void_p(_ptr(qkv)), ctypes.c_void_p(_ptr(q_norm_w)), ctypes.c_void_p(_ptr(k_norm_w)),
            ctypes.c_void_p(_ptr(cos)), ctypes.c_void_p(_ptr(sin)), ctypes.c_int32(P), ctypes.c_void_p(_ptr(q_out)),
            ctypes.c_void_p(_ptr(k_pool)), ctypes.c_void_p(_ptr(v_pool)), pool, ctypes.c_void_p(_ptr(block_tables)),
            ctypes.c_int32(int(block_tables.shape[1])), ctypes.c_void_p(_ptr(cu_seqlens_q)),
            ctypes.c_void_p(_ptr(pos_offsets)), ctypes.c_int32(B), ctypes.c_int32(T), ctypes.c_int32(num_q_heads),
            ctypes.c_float(eps), ctypes.c_int32(qk_mode), ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_split_qkv_norm_rope_into_paged_cache_varlen, args,
                        (qkv, q_norm_w, k_norm_w, cos, sin, q_out, k_pool, v_pool, block_tables, cu_seqlens_q,
                         pos_offsets))


def prepare_decode_step_qkv(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool, block_tables, context_lens,
                            num_q_heads: int, scale: float, eps: float, qk_mode: int, q_out, out, num_splits: int = 0,
                            max_context_hint: int = 0, stream=None) -> PreparedCall:
    """pkv_paged_decode_step_qkv with its arguments marshalled once (see PreparedCall)."""
    import torch
    _dev(out, torch.float16, "out", 3)
    pool, B, P = _step_qkv_args(qkv, q_norm_w, k_norm_w, cos, sin, k_pool, v_pool, block_tables, context_lens,
                                num_q_heads, qk_mode, q_out)
    lib = load()
    args = (ctypes.c_void_p(_ptr(qkv)), ctypes.c_void_p(_ptr(q_norm_w)), ctypes.c_void_p(_ptr(k_norm_w)),
            ctypes.c_void_p(_ptr(cos)), ctypes.c_void_p(_ptr(sin)), ctypes.c_int32(P), ctypes.c_float(eps),
            ctypes.c_int32(qk_mode), ctypes.c_void_p(_ptr(q_out)), ctypes.c_void_p(_ptr(k_pool)),
            ctypes.c_void_p(_ptr(v_pool)), pool, ctypes.c_void_p(_ptr(block_tables)),
            ctypes.c_int32(int(block_tables.shape[1])), ctypes.c_void_p(_ptr(context_lens)), ctypes.c_int32(B),
            ctypes.c_int32(num_q_heads), ctypes.c_float(scale), ctypes.c_void_p(_ptr(out)), ctypes.c_int32(num_splits),
            ctypes.c_int32(max_context_hint), ctypes.c_void_p(_stream(stream)))
    return PreparedCall(lib.pkv_paged_decode_step_qkv, args,
                        (qkv, q_norm_w, k_norm_w, cos, sin, q_out, k_pool, v_pool, block_tables, context_lens, out))
