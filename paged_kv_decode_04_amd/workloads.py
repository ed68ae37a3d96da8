"""Seeded synthetic inputs for paged-KV decode attention and the paged KV append.

The tests, the smoke check and the benchmark draw every input here, and the same host arrays feed both the HIP
library and the CPU oracle.  This module draws random numbers and builds index structures (context lengths, block
tables, slot mappings); it holds none of the attention arithmetic and imports neither the oracle nor the HIP binding.

Pool layouts, fixed by the library's header (each block is BS/16 panels of 16 rows):
    k_pool[N][Hkv][BS/16][D/32][16][32] fp16  (a panel holds each row's dims in 32-wide pieces, piece-major)
    v_pool[N][Hkv][BS/16][4][D][4] fp16     (a panel holds four quads of 4 rows, each dim's 4 rows adjacent)
Use k_row / v_row / set_k_row / set_v_row to address one token row.

Randomness: numpy PCG64 streams keyed by ``SeedSequence([seed, rotation, tag])``; large arrays are filled in fixed
chunks of ``_CHUNK`` elements, chunk c from ``SeedSequence([seed, rotation, tag, c])``, so the result does not depend
on the number of threads.  Values are drawn in float32 and rounded to fp16 (round to nearest even).

The five workloads mirror the shapes the pages' Llama-style models run (the pages publish no dataset or benchmark):
  c1  tiny:            B=1,   Hq=4,  Hkv=2,  D=64,  BS=16, L=37, pool of 8 blocks, table = 3 distinct ids
  c2  Llama-3-8B layer B=32,  Hq=32, Hkv=8,  D=128, BS=16, L ~ U{512..2048}
  c3  long context     B=4,   Hq=32, Hkv=8,  D=128, BS=16, L=32768, q ~ 2*N(0,1)
  c4  mixed serving    B=256, Hq=64, Hkv=8,  D=128, BS=16, L = clip(round(lognormal(ln 1024, 1)), 1, 16384)
  c5  MHA wide head    B=128, Hq=16, Hkv=16, D=256, BS=32, L=4096, K/V ~ U(-1,1), scale 1/16
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_CHUNK = 1 << 22
POISON = 60000.0  # fp16-representable marker for a row that the append must overwrite

SEEDS = {"c1": 0xC0FFEE01, "c2": 0xC0FFEE02, "c3": 0xC0FFEE03, "c4": 0xC0FFEE04, "c5": 0xC0FFEE05}

_TAGS = {"q": 1, "k": 2, "v": 3, "lens": 4, "perm": 5, "knew": 6, "vnew": 7, "choice": 8, "qkv": 9, "normw": 10}


def _rng(seed: int, rotation: int, tag: str, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, rotation, _TAGS[tag], *extra])))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fill_f16(out: np.ndarray, seed: int, rotation: int, tag: str, dist: str, scale: float = 1.0) -> np.ndarray:
    """Fill a C-contiguous float16 array in place with i.i.d. draws: dist 'normal' (N(0,1)) or 'uniform' (U(-1,1)),
    multiplied by ``scale`` in float32, then rounded to fp16."""
    if out.dtype != np.float16 or not out.flags.c_contiguous:
        raise ValueError("fill_f16 needs a C-contiguous float16 array")
    flat = out.reshape(-1)
    n = flat.size
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng = _rng(seed, rotation, tag, c)
        buf = np.empty(hi - lo, dtype=np.float32)
        if dist == "normal":
            rng.standard_normal(out=buf, dtype=np.float32)
        elif dist == "uniform":
            rng.random(out=buf, dtype=np.float32)
            buf *= np.float32(2.0)
            buf -= np.float32(1.0)
        else:
            raise ValueError(dist)
        if scale != 1.0:
            buf *= np.float32(scale)
        np.copyto(flat[lo:hi], buf, casting="same_kind")

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


@dataclass
class DecodeCase:
    """One decode step's inputs.  ``block_tables`` rows are padded with -1 past ceil(L/BS) entries."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    N: int
    M: int
    scale: float
    context_lens: np.ndarray           # [B] int32, rows including the newest token
    block_tables: np.ndarray           # [B][M] int32
    q: Optional[np.ndarray] = None      # [B][Hq][D] fp16
    k_pool: Optional[np.ndarray] = None  # [N][Hkv][BS/16][D/32][16][32] fp16
    v_pool: Optional[np.ndarray] = None  # [N][Hkv][BS/16][4][D][4] fp16
    k_new: Optional[np.ndarray] = None   # [T][Hkv][D] fp16, the rows appended this step
    v_new: Optional[np.ndarray] = None   # [T][Hkv][D] fp16
    slot_mapping: Optional[np.ndarray] = None  # [T] int32
    meta: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def num_tokens(self) -> int:
        return 0 if self.slot_mapping is None else int(self.slot_mapping.shape[0])


def carve_tables(context_lens: np.ndarray, BS: int, N: int, M: int, perm: np.ndarray) -> np.ndarray:
    """Block tables taken consecutively from a permutation of the pool's block ids; unused entries are -1."""
    B = context_lens.shape[0]
    bt = np.full((B, M), -1, dtype=np.int32)
    pos = 0
    for s in range(B):
        nb = (int(context_lens[s]) + BS - 1) // BS
        if nb > M:
            raise ValueError("sequence %d needs %d blocks > M=%d" % (s, nb, M))
        bt[s, :nb] = perm[pos:pos + nb]
        pos += nb
    if pos > N:
        raise ValueError("pool of %d blocks is too small for %d table entries" % (N, pos))
    return bt


def newest_row_slots(context_lens: np.ndarray, block_tables: np.ndarray, BS: int) -> np.ndarray:
    """Slot of each sequence's newest row (position L-1), as the callers on the pages form it:
    slot = block_tables[s][(L-1) / BS] * BS + (L-1) % BS; -1 for an empty sequence."""
    B = context_lens.shape[0]
    slots = np.full(B, -1, dtype=np.int32)
    for s in range(B):
        L = int(context_lens[s])
        if L > 0:
            slots[s] = int(block_tables[s, (L - 1) // BS]) * BS + (L - 1) % BS
    return slots


def poison_rows(k_pool: np.ndarray, v_pool: np.ndarray, slots: np.ndarray, BS: int) -> None:
    """Overwrite the pool rows at ``slots`` with POISON in every kv head and dim (layouts as in the module doc)."""
    for slot in slots:
        if slot < 0:
            continue
        b, o = int(slot) // BS, int(slot) % BS
        k_pool[b, :, o // 16, :, o % 16, :] = POISON
        v_pool[b, :, o // 16, (o % 16) // 4, :, o % 4] = POISON


def k_pool_shape(N: int, Hkv: int, BS: int, D: int) -> tuple:
    return (N, Hkv, BS // 16, D // 32, 16, 32)


def v_pool_shape(N: int, Hkv: int, BS: int, D: int) -> tuple:
    return (N, Hkv, BS // 16, 4, D, 4)


def _alloc_pools(N, Hkv, BS, D):
    if BS % 16 or D % 32:
        raise ValueError("block_size must be a multiple of 16 and head_dim a multiple of 32")
    return (np.empty(k_pool_shape(N, Hkv, BS, D), dtype=np.float16),
            np.empty(v_pool_shape(N, Hkv, BS, D), dtype=np.float16))


def k_row(k_pool: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    """The D values of K row `offset` of (block, head), read through the panel layout."""
    return k_pool[block, head, offset // 16, :, offset % 16, :].reshape(-1)


def v_row(v_pool: np.ndarray, block: int, head: int, offset: int) -> np.ndarray:
    return v_pool[block, head, offset // 16, (offset % 16) // 4, :, offset % 4]


def set_k_row(k_pool: np.ndarray, block: int, head, offset: int, row) -> None:
    """Write K row(s) of D values at (block, head(s), offset)."""
    r = np.asarray(row, dtype=np.float16)
    k_pool[block, head, offset // 16, :, offset % 16, :] = r.reshape(r.shape[:-1] + (-1, 32))


def set_v_row(v_pool: np.ndarray, block: int, head, offset: int, row) -> None:
    v_pool[block, head, offset // 16, (offset % 16) // 4, :, offset % 4] = np.asarray(row, dtype=np.float16)


def build_case(name: str, B: int, Hq: int, Hkv: int, D: int, BS: int, context_lens, N: int, M: int, scale: float,
               seed: int, rotation: int = 0, q_scale: float = 1.0, kv_dist: str = "normal",
               with_append: bool = True, poison: bool = False, table_ids: Optional[np.ndarray] = None,
               with_pools: bool = True) -> DecodeCase:
    """General builder: pools filled i.i.d., tables carved from a seeded permutation of the N block ids (or given),
    one appended token per non-empty sequence at its newest row when ``with_append``.  ``with_pools=False`` builds
    only the lengths, tables and slot mapping (q, pools and new rows stay None)."""
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    if table_ids is None:
        perm = _rng(seed, rotation, "perm").permutation(N).astype(np.int32)
    else:
        perm = np.asarray(table_ids, dtype=np.int32)
    bt = carve_tables(cl, BS, N, M, perm)
    if not with_pools:
        case = DecodeCase(name, B, Hq, Hkv, D, BS, N, M, float(scale), cl, bt)
        if with_append:
            slots = newest_row_slots(cl, bt, BS)
            case.slot_mapping = np.ascontiguousarray(slots[slots >= 0])
        return case
    q = fill_f16(np.empty((B, Hq, D), dtype=np.float16), seed, rotation, "q", "normal", q_scale)
    k_pool, v_pool = _alloc_pools(N, Hkv, BS, D)
    fill_f16(k_pool, seed, rotation, "k", kv_dist)
    fill_f16(v_pool, seed, rotation, "v", kv_dist)
    case = DecodeCase(name, B, Hq, Hkv, D, BS, N, M, float(scale), cl, bt, q, k_pool, v_pool)
    if with_append:
        slots = newest_row_slots(cl, bt, BS)
        keep = slots >= 0
        slots = np.ascontiguousarray(slots[keep])
        T = int(slots.shape[0])
        case.k_new = fill_f16(np.empty((T, Hkv, D), dtype=np.float16), seed, rotation, "knew", kv_dist)
        case.v_new = fill_f16(np.empty((T, Hkv, D), dtype=np.float16), seed, rotation, "vnew", kv_dist)
        case.slot_mapping = slots
        if poison:
            poison_rows(k_pool, v_pool, slots, BS)
    return case


def pool_blocks_for(context_lens: np.ndarray, BS: int, extra: float = 0.10) -> int:
    """Pool size = ceil((1 + extra) * sum of per-sequence blocks)."""
    total = int(sum((int(L) + BS - 1) // BS for L in context_lens))
    return int(math.ceil((1.0 + extra) * total))


def config_c1(rotation: int = 0, with_pools: bool = True) -> DecodeCase:
    """B=1, 4/2 heads, D=64, BS=16, L=37, pool of 8 blocks, table = 3 distinct seeded ids; one appended token.

    The appended token is the sequence's newest row, position 36 = L-1, written through the table
    (slot = bt[0][2]*16 + 4)."""
    seed = SEEDS["c1"]
    ids = _rng(seed, rotation, "choice").choice(8, size=3, replace=False).astype(np.int32)
    return build_case("c1", 1, 4, 2, 64, 16, [37], 8, 3, 1.0 / 8.0, seed, rotation, table_ids=ids, poison=True,
                      with_pools=with_pools)


def config_c2(rotation: int = 0, with_pools: bool = True) -> DecodeCase:
    """Llama-3-8B-shaped layer: B=32, 32/8 heads, D=128, BS=16, L ~ U{512..2048}, pool = blocks + 10%, M=128."""
    seed = SEEDS["c2"]
    lens = _rng(seed, rotation, "lens").integers(512, 2048, size=32, endpoint=True).astype(np.int32)
    N = pool_blocks_for(lens, 16)
    return build_case("c2", 32, 32, 8, 128, 16, lens, N, 128, 1.0 / math.sqrt(128.0), seed, rotation, poison=True,
                      with_pools=with_pools)


def config_c3(rotation: int = 0, with_pools: bool = True) -> DecodeCase:
    """Long context: B=4, 32/8 heads, D=128, BS=16, L=32768, N=8192, M=2048, q ~ 2*N(0,1)."""
    seed = SEEDS["c3"]
    lens = np.full(4, 32768, dtype=np.int32)
    return build_case("c3", 4, 32, 8, 128, 16, lens, 8192, 2048, 1.0 / math.sqrt(128.0), seed, rotation,
                      q_scale=2.0, poison=True, with_pools=with_pools)


def c4_context_lens(rotation: int = 0) -> np.ndarray:
    seed = SEEDS["c4"]
    raw = _rng(seed, rotation, "lens").lognormal(mean=math.log(1024.0), sigma=1.0, size=256)
    return np.clip(np.rint(raw), 1, 16384).astype(np.int32)


def config_c4(rotation: int = 0, with_pools: bool = True) -> DecodeCase:
    """Mixed serving batch: B=256, 64/8 heads, D=128, BS=16, lognormal lengths (median 1024, sigma 1, clipped
    to [1, 16384]); the newest row of every sequence is poisoned, then re-written by the append."""
    seed = SEEDS["c4"]
    lens = c4_context_lens(rotation)
    N = pool_blocks_for(lens, 16)
    M = int((int(lens.max()) + 15) // 16)
    return build_case("c4", 256, 64, 8, 128, 16, lens, N, M, 1.0 / math.sqrt(128.0), seed, rotation, poison=True,
                      with_pools=with_pools)


def config_c5(rotation: int = 0, with_pools: bool = True) -> DecodeCase:
    """MHA wide head: B=128, 16/16 heads, D=256, BS=32, L=4096, N=16384, M=128, K/V ~ U(-1,1), q ~ N(0,1),
    scale = 1/16."""
    seed = SEEDS["c5"]
    lens = np.full(128, 4096, dtype=np.int32)
    return build_case("c5", 128, 16, 16, 256, 32, lens, 16384, 128, 1.0 / 16.0, seed, rotation,
                      kv_dist="uniform", poison=True, with_pools=with_pools)


CONFIGS = {"c1": config_c1, "c2": config_c2, "c3": config_c3, "c4": config_c4, "c5": config_c5}


def small_case(seed: int, B: int, Hq: int, Hkv: int, D: int, BS: int, lens, extra_blocks: int = 3,
               q_scale: float = 1.0, kv_dist: str = "normal", scale: Optional[float] = None,
               poison: bool = False, M: Optional[int] = None) -> DecodeCase:
    """A reduced case of the same structure for parity tests the oracle finishes in seconds."""
    lens = np.asarray(lens, dtype=np.int32)
    nbs = [(int(L) + BS - 1) // BS for L in lens]
    N = sum(nbs) + extra_blocks
    if M is None:
        M = max(1, max(nbs) if nbs else 1)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return build_case("small", int(B), Hq, Hkv, D, BS, lens, N, M, scale, seed, 0, q_scale=q_scale,
                      kv_dist=kv_dist, poison=poison)


def algorithmic_bytes(case: DecodeCase, window: int = 0) -> dict:
    """Bytes a decode step must move at minimum: K and V rows actually used (with a sliding window W > 0, each
    sequence's last W rows), q, out, tables and lengths; the append reads and writes 2*T*Hkv*D fp16 values."""
    lens = np.maximum(case.context_lens, 0)
    if window > 0:
        lens = np.minimum(lens, window)
    rows = int(lens.sum())
    kv = rows * case.Hkv * case.D * 2 * 2
    qo = 2 * case.B * case.Hq * case.D * 2
    nb = int(sum((int(L) + case.BS - 1) // case.BS for L in lens))
    idx = nb * 4 + case.B * 4
    app = 2 * 2 * case.num_tokens * case.Hkv * case.D * 2 + case.num_tokens * 4
    return {"kv": kv, "q_out": qo, "index": idx, "attention": kv + qo + idx, "append": app}


@dataclass
class VarlenCase:
    """Inputs of paged varlen attention: sequence s owns the query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1
    (token-major q[T][Hq][D]); its i-th new row sits at position pos_offsets[s] + i.  The new rows' K/V
    (k_new / v_new, at slot_mapping) are written into the pools before attention; with ``poison_new`` the pools hold
    POISON there until that append.  Rows of a sequence's last block past its final length hold POISON."""
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    N: int
    M: int
    scale: float
    q_lens: np.ndarray        # [B] int32
    pos_offsets: np.ndarray   # [B] int32
    cu_seqlens_q: np.ndarray  # [B+1] int32
    block_tables: np.ndarray  # [B][M] int32, -1 past the used entries
    q: np.ndarray             # [T][Hq][D] fp16
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_new: np.ndarray         # [T][Hkv][D] fp16
    v_new: np.ndarray
    slot_mapping: np.ndarray  # [T] int32

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def T(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def final_lens(self) -> np.ndarray:
        return (self.pos_offsets + self.q_lens).astype(np.int32)


def build_varlen_case(name: str, B: int, Hq: int, Hkv: int, D: int, BS: int, q_lens, pos_offsets, seed: int,
                      rotation: int = 0, extra_blocks: int = 3, scale: Optional[float] = None, q_scale: float = 1.0,
                      kv_dist: str = "normal", poison_new: bool = True, M: Optional[int] = None) -> VarlenCase:
    ql = np.ascontiguousarray(np.asarray(q_lens, dtype=np.int32))
    po = np.ascontiguousarray(np.asarray(pos_offsets, dtype=np.int32))
    final = ql + po
    nbs = (final + BS - 1) // BS
    if M is None:
        M = max(1, int(nbs.max()) if B else 1)
    N = int(nbs.sum()) + extra_blocks
    perm = _rng(seed, rotation, "perm").permutation(N).astype(np.int32)
    bt = carve_tables(final, BS, N, M, perm)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ql)
    T = int(cu[-1])
    q = fill_f16(np.empty((max(T, 0), Hq, D), dtype=np.float16), seed, rotation, "q", "normal", q_scale)
    k_pool, v_pool = _alloc_pools(N, Hkv, BS, D)
    fill_f16(k_pool, seed, rotation, "k", kv_dist)
    fill_f16(v_pool, seed, rotation, "v", kv_dist)
    k_new = fill_f16(np.empty((T, Hkv, D), dtype=np.float16), seed, rotation, "knew", kv_dist)
    v_new = fill_f16(np.empty((T, Hkv, D), dtype=np.float16), seed, rotation, "vnew", kv_dist)
    slots = np.empty(T, dtype=np.int32)
    for s in range(B):
        for i in range(int(ql[s])):
            t = int(po[s]) + i
            slots[cu[s] + i] = int(bt[s, t // BS]) * BS + t % BS
    tail = []
    for s in range(B):
        for t in range(int(final[s]), int(nbs[s]) * BS):
            tail.append(int(bt[s, t // BS]) * BS + t % BS)
    poison_rows(k_pool, v_pool, np.asarray(tail, dtype=np.int64), BS)
    if poison_new:
        poison_rows(k_pool, v_pool, slots, BS)
    else:
        for j, slot in enumerate(slots):
            b, o = int(slot) // BS, int(slot) % BS
            set_k_row(k_pool, b, slice(None), o, k_new[j])
            set_v_row(v_pool, b, slice(None), o, v_new[j])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return VarlenCase(name, B, Hq, Hkv, D, BS, N, M, float(scale), ql, po, cu, bt, q, k_pool, v_pool, k_new, v_new,
                      slots)


SEEDS["v1"] = 0xC0FFEE11


def config_v1(rotation: int = 0) -> VarlenCase:
    """Speculative verification on the Llama-3-8B-shaped batch: B=32, 32/8 heads, D=128, BS=16, 4 new rows per
    sequence whose final lengths are U{512..2048} (positions L-4 .. L-1), pool = blocks + 10%.  The new rows are
    poisoned in the pools until the step's append writes them."""
    seed = SEEDS["v1"]
    final = _rng(seed, rotation, "lens").integers(512, 2048, size=32, endpoint=True).astype(np.int32)
    ql = np.full(32, 4, dtype=np.int32)
    nblocks = int(sum((int(L) + 15) // 16 for L in final))
    return build_varlen_case("v1", 32, 32, 8, 128, 16, ql, final - ql, seed, rotation,
                             extra_blocks=int(math.ceil(0.10 * nblocks)), M=128)


SEEDS["v2"] = 0xC0FFEE12


def config_v2(rotation: int = 0) -> VarlenCase:
    """Speculative verification of 8 draft tokens on the Llama-3-8B-shaped batch: B=32, 32/8 heads, D=128, BS=16,
    8 new rows per sequence whose final lengths are U{512..2048}, pool = blocks + 10%."""
    seed = SEEDS["v2"]
    final = _rng(seed, rotation, "lens").integers(512, 2048, size=32, endpoint=True).astype(np.int32)
    ql = np.full(32, 8, dtype=np.int32)
    nblocks = int(sum((int(L) + 15) // 16 for L in final))
    return build_varlen_case("v2", 32, 32, 8, 128, 16, ql, final - ql, seed, rotation,
                             extra_blocks=int(math.ceil(0.10 * nblocks)), M=128)


SEEDS["v3"] = 0xC0FFEE13


def config_v3(rotation: int = 0) -> VarlenCase:
    """Speculative verification on the mixed serving batch: B=256, 64/8 heads, D=128, BS=16, 4 new rows per
    sequence whose final lengths are drawn as c4's (lognormal, median 1024, sigma 1, clipped to [4, 16384]), pool =
    blocks + 10% (2048 workgroups: several rounds of the CUs)."""
    seed = SEEDS["v3"]
    raw = _rng(seed, rotation, "lens").lognormal(mean=math.log(1024.0), sigma=1.0, size=256)
    final = np.clip(np.rint(raw), 4, 16384).astype(np.int32)
    ql = np.full(256, 4, dtype=np.int32)
    nblocks = int(sum((int(L) + 15) // 16 for L in final))
    return build_varlen_case("v3", 256, 64, 8, 128, 16, ql, final - ql, seed, rotation,
                             extra_blocks=int(math.ceil(0.10 * nblocks)))


VARLEN_CONFIGS = {"v1": config_v1, "v2": config_v2, "v3": config_v3}


def algorithmic_bytes_varlen(case: VarlenCase) -> dict:
    """Bytes a varlen step must move at minimum: each sequence's K and V rows up to its final length read once
    (every tile of new rows shares them), q and out, tables, prefix sums and positions; the append reads and writes
    2*T*Hkv*D fp16 values."""
    final = case.final_lens
    kv = int(final.sum()) * case.Hkv * case.D * 2 * 2
    qo = 2 * case.T * case.Hq * case.D * 2
    nb = int(sum((int(L) + case.BS - 1) // case.BS for L in final))
    idx = nb * 4 + (2 * case.B + 1) * 4
    app = 2 * 2 * case.T * case.Hkv * case.D * 2 + case.T * 4
    return {"kv": kv, "q_out": qo, "index": idx, "attention": kv + qo + idx, "append": app}


def rope_tables(num_positions: int, head_dim: int, theta: float):
    """cos and sin tables [num_positions][head_dim/2] float32 of the usual rotary frequencies: entry (p, j) is the
    angle p * theta^(-2j/head_dim), evaluated in float64 and rounded once.  These are the caller's tables (a model's
    configuration), inputs to the QKV step."""
    half = head_dim // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=np.float64) / head_dim)
    ang = np.arange(num_positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


@dataclass
class QkvCase:
    """Inputs of the QKV-to-cache step followed by attention.  ``qkv`` [T][(Hq + 2*Hkv)*D] fp16 holds each new
    token's query heads, key heads and value heads; ``varlen`` carries the batch geometry (sequences, new rows at
    positions pos_offsets[s] + i, block tables, pools whose new rows hold POISON until the step writes them)."""
    name: str
    varlen: VarlenCase
    qkv: np.ndarray
    q_norm_w: np.ndarray   # [D] fp16
    k_norm_w: np.ndarray   # [D] fp16
    cos: np.ndarray        # [P][D/2] float32
    sin: np.ndarray
    eps: float
    qk_mode: int


def build_qkv_case(name: str, B: int, Hq: int, Hkv: int, D: int, BS: int, q_lens, pos_offsets, seed: int,
                   qk_mode: int = 1, eps: float = 1e-6, theta: float = 1.0e6, qkv_scale: float = 1.0,
                   rotation: int = 0, extra_blocks: int = 3, M: Optional[int] = None,
                   num_positions: Optional[int] = None) -> QkvCase:
    """qkv ~ qkv_scale * N(0,1), norm weights ~ 1 + 0.25 * N(0,1) (both rounded to fp16), rotary tables for
    ``theta`` covering every position the batch reaches (or ``num_positions`` rows)."""
    vc = build_varlen_case(name, B, Hq, Hkv, D, BS, q_lens, pos_offsets, seed, rotation, extra_blocks=extra_blocks,
                           poison_new=True, M=M)
    T = vc.T
    qkv = fill_f16(np.empty((T, (Hq + 2 * Hkv) * D), dtype=np.float16), seed, rotation, "qkv", "normal", qkv_scale)
    rng = _rng(seed, rotation, "normw")
    w = (1.0 + 0.25 * rng.standard_normal((2, D), dtype=np.float32)).astype(np.float16)
    if num_positions is None:
        num_positions = max(1, int(vc.final_lens.max()) if B else 1)
    cos, sin = rope_tables(num_positions, D, theta)
    return QkvCase(name, vc, qkv, np.ascontiguousarray(w[0]), np.ascontiguousarray(w[1]), cos, sin, float(eps),
                   int(qk_mode))


SEEDS["r1"] = 0xC0FFEE21
SEEDS["r2"] = 0xC0FFEE22


def config_r1(rotation: int = 0) -> QkvCase:
    """Decode step of a Qwen3-8B-shaped layer (32/8 heads, D=128, q/k RMSNorm): B=32, BS=16, one new token per
    sequence whose final lengths are U{512..2048} as in the Llama-3-8B-shaped batch, pool = blocks + 10%, M=128,
    rotary theta 1e6, eps 1e-6.  The QKV step writes q and the new K/V rows, then single-pass attention reads
    them."""
    seed = SEEDS["r1"]
    final = _rng(seed, rotation, "lens").integers(512, 2048, size=32, endpoint=True).astype(np.int32)
    ql = np.ones(32, dtype=np.int32)
    nblocks = int(sum((int(L) + 15) // 16 for L in final))
    return build_qkv_case("r1", 32, 32, 8, 128, 16, ql, final - ql, seed, qk_mode=1,
                          extra_blocks=int(math.ceil(0.10 * nblocks)), M=128, rotation=rotation)


def config_r2(rotation: int = 0) -> QkvCase:
    """Chunked prefill of the same layer: B=4 sequences each adding 512 new rows after a cached prefix of
    U{0..1024} rows (so chunks start mid-block), BS=16, pool = blocks + 10%.  The QKV step writes 2048 tokens'
    q and K/V rows, then varlen attention reads them."""
    seed = SEEDS["r2"]
    pre = _rng(seed, rotation, "lens").integers(0, 1024, size=4, endpoint=True).astype(np.int32)
    ql = np.full(4, 512, dtype=np.int32)
    final = pre + ql
    nblocks = int(sum((int(L) + 15) // 16 for L in final))
    return build_qkv_case("r2", 4, 32, 8, 128, 16, ql, pre, seed, qk_mode=1,
                          extra_blocks=int(math.ceil(0.10 * nblocks)), rotation=rotation)


QKV_CONFIGS = {"r1": config_r1, "r2": config_r2}


def algorithmic_bytes_qkv(case: QkvCase) -> int:
    """Bytes the QKV step must move at minimum: the qkv rows read, q written, the new K and V rows written, the norm
    weights and each token's cos/sin row read, tables and positions."""
    vc = case.varlen
    T, D = vc.T, vc.D
    qkv = T * (vc.Hq + 2 * vc.Hkv) * D * 2
    q_out = T * vc.Hq * D * 2
    kv = 2 * T * vc.Hkv * D * 2
    rope = 2 * T * (D // 2) * 4
    idx = (2 * vc.B + 1) * 4 + T * 4
    return qkv + q_out + kv + rope + 2 * D * 2 + idx
