"""Pins for the CPU oracle (runs without a GPU).

The oracle is checked against things other than itself: hand-derived fixtures (tests/golden/), closed forms
(single row, constant V, scale 0, dominant key), invariants (weights sum to 1, block-id permutation), a contiguous
brute force written here in numpy from rows generated before they are scattered into the pool, torch's CPU
scaled_dot_product_attention in float64 (a library routine), numpy's own fp16 decoding and array strides.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, str):
        table = {"ln3": math.log(3.0), "-ln3": -math.log(3.0), "ln2": math.log(2.0), "nan": float("nan")}
        return table[x]
    return float(x)


def _nums(a):
    if isinstance(a, list):
        return [_nums(x) for x in a]
    return _num(a)


def _pad32(x, D):
    """Zero-pad the last axis from D to the next multiple of 32 (the K layout needs D % 32 == 0); zero dims change
    no dot product, and the outputs on them are sums of zeros."""
    x = np.asarray(x, dtype=np.float64)
    Dp = (D + 31) // 32 * 32
    pad = [(0, 0)] * (x.ndim - 1) + [(0, Dp - D)]
    return np.pad(x, pad)


def _zero_pools(N, Hkv, BS, D):
    return (np.zeros(W.k_pool_shape(N, Hkv, BS, D), dtype=np.float16),
            np.zeros(W.v_pool_shape(N, Hkv, BS, D), dtype=np.float16))


def _pools_from_rows(case):
    N, Hkv, BS, D = case["N"], case["Hkv"], case["BS"], case["D"]
    Dp = (D + 31) // 32 * 32
    k_pool, v_pool = _zero_pools(N, Hkv, BS, Dp)
    for r in case["rows"]:
        W.set_k_row(k_pool, r["block"], r["head"], r["offset"], _pad32(r["k"], D))
        W.set_v_row(v_pool, r["block"], r["head"], r["offset"], _pad32(r["v"], D))
    return k_pool, v_pool


# --------------------------------------------------------------------------------------------------------------
# fp16 decoding and pool layout


def test_f16_decode_matches_numpy_on_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_pool_index_functions_match_numpy_strides():
    rng = np.random.default_rng(7)
    for (N, Hkv, BS, D) in [(5, 3, 16, 64), (2, 1, 32, 256), (7, 8, 16, 128), (3, 2, 64, 32)]:
        k = np.empty(W.k_pool_shape(N, Hkv, BS, D), dtype=np.float16)
        v = np.empty(W.v_pool_shape(N, Hkv, BS, D), dtype=np.float16)
        for _ in range(50):
            b, h, o, d = (int(rng.integers(N)), int(rng.integers(Hkv)), int(rng.integers(BS)), int(rng.integers(D)))
            assert oracle.k_index(Hkv, BS, D, b, h, o, d) * 2 == np.dot(k.strides, (b, h, o // 16, d // 32, o % 16, d % 32))
            assert oracle.v_index(Hkv, BS, D, b, h, o, d) * 2 == np.dot(v.strides,
                                                                        (b, h, o // 16, (o % 16) // 4, d, o % 4))


def test_row_helpers_round_trip():
    rng = np.random.default_rng(8)
    k, v = _zero_pools(3, 2, 32, 32)
    row = rng.standard_normal(32).astype(np.float16)
    W.set_k_row(k, 1, 1, 21, row)
    W.set_v_row(v, 1, 1, 21, row)
    assert np.array_equal(W.k_row(k, 1, 1, 21), row) and np.array_equal(W.v_row(v, 1, 1, 21), row)
    assert np.count_nonzero(k) == np.count_nonzero(row) == np.count_nonzero(v)
    for d in range(32):
        assert k.reshape(-1)[oracle.k_index(2, 32, 32, 1, 1, 21, d)] == row[d]
        assert v.reshape(-1)[oracle.v_index(2, 32, 32, 1, 1, 21, d)] == row[d]


# --------------------------------------------------------------------------------------------------------------
# hand-derived fixtures


def _golden_attention_cases():
    with open(os.path.join(GOLDEN, "attention_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_attention_cases(), ids=lambda c: c["name"])
def test_golden_attention(case):
    k_pool, v_pool = _pools_from_rows(case)
    q = _pad32(case["q"], case["D"]).astype(np.float16)
    bt = np.array(case["block_tables"], dtype=np.int32)
    cl = np.array(case["context_lens"], dtype=np.int32)
    scale = _num(case["scale"])
    out = oracle.decode_attention(q, k_pool, v_pool, bt, cl, scale, threads=2)
    np.testing.assert_allclose(out, _pad32(case["expected"], case["D"]), rtol=1e-14, atol=1e-14)
    if "weights" in case:
        for s, wexp in enumerate(case["weights"]):
            _, w = oracle.attention_weights(q, k_pool, v_pool, bt, cl, scale, s, 0)
            np.testing.assert_allclose(w, wexp, rtol=1e-14, atol=1e-15)


def _golden_combine_cases():
    with open(os.path.join(GOLDEN, "split_combine_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_combine_cases(), ids=lambda c: c["name"])
def test_golden_split_combine(case):
    O = np.array(_nums(case["O"]), dtype=np.float64)
    m = np.array(_nums(case["m"]), dtype=np.float64)
    l = np.array(_nums(case["l"]), dtype=np.float64)
    out = oracle.split_combine(O, m, l, case["context_lens"], case["BS"], case["chunk_blocks"])
    if "expected" in case:
        expected = np.array(case["expected"])
    else:
        expected = np.array(eval(case["expected_formula"], {"exp": math.exp}))
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out.reshape(-1), np.reshape(expected, -1), rtol=1e-14)


def test_golden_append():
    with open(os.path.join(GOLDEN, "append_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        N, Hkv, BS, D = c["N"], c["Hkv"], c["BS"], c["D"]
        k_pool, v_pool = _zero_pools(N, Hkv, BS, (D + 31) // 32 * 32)
        skipped = oracle.paged_kv_append(_pad32(c["k"], D).astype(np.float16), _pad32(c["v"], D).astype(np.float16),
                                         c["slot_mapping"], k_pool, v_pool)
        assert skipped == c["expected_skipped"]
        k_exp = np.zeros_like(k_pool)
        v_exp = np.zeros_like(v_pool)
        for r in c["expected_rows"]:
            W.set_k_row(k_exp, r["block"], r["head"], r["offset"], _pad32(r["k"], D))
            W.set_v_row(v_exp, r["block"], r["head"], r["offset"], _pad32(r["v"], D))
        assert np.array_equal(k_pool, k_exp)
        assert np.array_equal(v_pool, v_exp)


# --------------------------------------------------------------------------------------------------------------
# closed forms and invariants on random inputs


def _rand_case(seed, B=3, Hq=8, Hkv=2, D=64, BS=16, lens=(37, 16, 5), **kw):
    return W.small_case(seed, B, Hq, Hkv, D, BS, lens, **kw)


def _run(c, scale=None, q=None):
    return oracle.decode_attention(c.q if q is None else q, c.k_pool, c.v_pool, c.block_tables, c.context_lens,
                                   c.scale if scale is None else scale, threads=4)


def _rows(c, s, hk):
    """K and V rows of (s, kv head hk) in order, gathered with numpy indexing on the pool arrays."""
    L = int(c.context_lens[s])
    ks, vs = [], []
    for t in range(L):
        b = int(c.block_tables[s, t // c.BS])
        ks.append(W.k_row(c.k_pool, b, hk, t % c.BS).astype(np.float64))
        vs.append(W.v_row(c.v_pool, b, hk, t % c.BS).astype(np.float64))
    return np.array(ks).reshape(L, c.D), np.array(vs).reshape(L, c.D)


def test_single_row_context_returns_v0_exactly():
    c = _rand_case(11, lens=(1, 1, 1))
    out = _run(c)
    for s in range(c.B):
        for hq in range(c.Hq):
            _, v = _rows(c, s, hq // c.G)
            assert np.array_equal(out[s, hq], v[0])


def test_constant_v_returns_the_constant():
    c = _rand_case(12, lens=(37, 100, 3))
    for val in (0.5, -3.25, 7.0):
        c.v_pool[...] = np.float16(val)
        out = _run(c)
        np.testing.assert_allclose(out, val, rtol=1e-15, atol=0)


def test_weights_sum_to_one_and_are_nonnegative():
    c = _rand_case(13, lens=(37, 300, 5), q_scale=3.0)
    for s in range(c.B):
        for hq in (0, c.Hq - 1):
            out, w = oracle.attention_weights(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                                              s, hq)
            assert w.shape == (int(c.context_lens[s]),)
            assert np.all(w >= 0)
            assert abs(w.sum() - 1.0) < 1e-12
            _, v = _rows(c, s, hq // c.G)
            np.testing.assert_allclose(out, w @ v, rtol=1e-12, atol=1e-13)


def test_block_id_permutation_leaves_output_bitwise_identical():
    c = _rand_case(14, lens=(37, 64, 129), extra_blocks=5)
    ref = _run(c)
    rng = np.random.default_rng(99)
    for _ in range(3):
        perm = rng.permutation(c.N)  # new id of old block b is perm[b]
        k2 = np.empty_like(c.k_pool)
        v2 = np.empty_like(c.v_pool)
        k2[perm] = c.k_pool
        v2[perm] = c.v_pool
        bt2 = np.where(c.block_tables >= 0, perm[np.maximum(c.block_tables, 0)], -1).astype(np.int32)
        out = oracle.decode_attention(c.q, k2, v2, bt2, c.context_lens, c.scale, threads=3)
        assert np.array_equal(out.view(np.uint64), ref.view(np.uint64))


def test_scale_zero_and_zero_query_give_the_mean_of_v():
    c = _rand_case(15, lens=(37, 20, 2))
    out0 = _run(c, scale=0.0)
    outq = _run(c, q=np.zeros_like(c.q))
    for s in range(c.B):
        for hq in range(c.Hq):
            _, v = _rows(c, s, hq // c.G)
            np.testing.assert_allclose(out0[s, hq], v.mean(axis=0), rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(outq[s, hq], v.mean(axis=0), rtol=1e-13, atol=1e-14)


def test_one_dominant_key_returns_its_value():
    c = _rand_case(16, B=1, Hq=2, Hkv=1, lens=(50,))
    s, target = 0, 23
    b = int(c.block_tables[s, target // c.BS])
    q = np.zeros_like(c.q)
    q[s, :, 0] = np.float16(64.0)
    c.k_pool[...] = np.float16(0.0)
    row = np.zeros(c.D, np.float16)
    row[0] = 64.0  # z = 64 * 64 * scale = 512 against 0 for every other row
    W.set_k_row(c.k_pool, b, 0, target % c.BS, row)
    out = _run(c, q=q)
    _, v = _rows(c, s, 0)
    np.testing.assert_allclose(out[s, 0], v[target], rtol=1e-15, atol=1e-15)


def test_empty_sequence_gives_zero():
    c = _rand_case(17, lens=(0, 5, 0))
    out = _run(c)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.any(out[1] != 0)


def test_bad_table_entry_is_an_error():
    c = _rand_case(18, lens=(37, 5, 5))
    c.block_tables[0, 1] = c.N  # outside the pool
    with pytest.raises(ValueError):
        _run(c)


# --------------------------------------------------------------------------------------------------------------
# contiguous brute force and a library routine


def _contiguous_problem(seed, B, Hq, Hkv, D, BS, lens, scale):
    """Rows are drawn contiguous per (sequence, kv head) first, then scattered into a pool through a random table;
    the oracle must gather them back."""
    rng = np.random.default_rng(seed)
    G = Hq // Hkv
    nbs = [(L + BS - 1) // BS for L in lens]
    N = sum(nbs) + 4
    M = max(nbs)
    perm = rng.permutation(N).astype(np.int32)
    bt = np.full((B, M), -1, np.int32)
    k_pool = rng.standard_normal(W.k_pool_shape(N, Hkv, BS, D)).astype(np.float16)
    v_pool = rng.standard_normal(W.v_pool_shape(N, Hkv, BS, D)).astype(np.float16)
    q = rng.standard_normal((B, Hq, D)).astype(np.float16)
    Kc, Vc = [], []
    pos = 0
    for s, L in enumerate(lens):
        bt[s, :nbs[s]] = perm[pos:pos + nbs[s]]
        pos += nbs[s]
        ks = rng.standard_normal((Hkv, L, D)).astype(np.float16)
        vs = rng.standard_normal((Hkv, L, D)).astype(np.float16)
        for t in range(L):
            b = bt[s, t // BS]
            W.set_k_row(k_pool, b, slice(None), t % BS, ks[:, t, :])
            W.set_v_row(v_pool, b, slice(None), t % BS, vs[:, t, :])
        Kc.append(ks)
        Vc.append(vs)
    return q, k_pool, v_pool, bt, np.array(lens, np.int32), Kc, Vc, G


@pytest.mark.parametrize("geom", [
    (2, 4, 2, 64, 16, (37, 90), 0.125),
    (3, 8, 1, 128, 16, (1, 17, 48), 1 / math.sqrt(128)),
    (2, 4, 4, 256, 32, (33, 70), 1 / 16),
    (1, 16, 2, 32, 64, (90,), 0.3),
])
def test_paged_equals_contiguous_brute_force_and_torch_sdpa(geom):
    import torch
    B, Hq, Hkv, D, BS, lens, scale = geom
    q, k_pool, v_pool, bt, cl, Kc, Vc, G = _contiguous_problem(1234 + D + B, B, Hq, Hkv, D, BS, lens, scale)
    out = oracle.decode_attention(q, k_pool, v_pool, bt, cl, scale, threads=2)
    for s in range(B):
        for hq in range(Hq):
            K = Kc[s][hq // G].astype(np.float64)
            V = Vc[s][hq // G].astype(np.float64)
            z = scale * (K @ q[s, hq].astype(np.float64))
            w = np.exp(z - z.max())
            w /= w.sum()
            np.testing.assert_allclose(out[s, hq], w @ V, rtol=1e-12, atol=1e-13)
        Kt = torch.from_numpy(Kc[s].astype(np.float64)).repeat_interleave(G, dim=0)  # [Hq][L][D]
        Vt = torch.from_numpy(Vc[s].astype(np.float64)).repeat_interleave(G, dim=0)
        qt = torch.from_numpy(q[s].astype(np.float64)).unsqueeze(1)  # [Hq][1][D]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale).squeeze(1).numpy()
        np.testing.assert_allclose(out[s], ref, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------------------------------------------
# split-K emulation and the combine


@pytest.mark.parametrize("S,chunk", [(1, 0), (2, 0), (3, 0), (8, 0), (16, 0), (32, 0), (20, 1), (7, 3), (40, 2)])
def test_split_partials_then_combine_equal_dense(S, chunk):
    c = _rand_case(21, B=4, lens=(37, 300, 1, 0), q_scale=2.0)
    dense = _run(c)
    nbmax = max((int(L) + c.BS - 1) // c.BS for L in c.context_lens)
    if chunk and S * chunk < nbmax:
        pytest.skip("grid too small for this chunk")
    O, m, l = oracle.split_partials(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale, S, chunk)
    out = oracle.split_combine(O, m, l, c.context_lens, c.BS, chunk)
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-13)


def test_split_partials_match_their_definition_on_each_range():
    c = _rand_case(22, B=2, Hq=4, Hkv=2, lens=(100, 33))
    S = 3
    O, m, l = oracle.split_partials(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale, S)
    for s in range(c.B):
        L = int(c.context_lens[s])
        nb = (L + c.BS - 1) // c.BS
        chunk = (nb + S - 1) // S
        for hq in range(c.Hq):
            K, V = _rows(c, s, hq // c.G)
            z = c.scale * (K @ c.q[s, hq].astype(np.float64))
            for j in range(S):
                t0, t1 = j * chunk * c.BS, min(L, (j + 1) * chunk * c.BS)
                if t1 <= t0:
                    assert m[s, hq, j] == -np.inf and l[s, hq, j] == 0 and np.all(O[s, hq, j] == 0)
                    continue
                mj = z[t0:t1].max()
                e = np.exp(z[t0:t1] - mj)
                assert abs(m[s, hq, j] - mj) <= 1e-15 * max(1, abs(mj))
                np.testing.assert_allclose(l[s, hq, j], e.sum(), rtol=1e-13)
                np.testing.assert_allclose(O[s, hq, j], e @ V[t0:t1], rtol=1e-12, atol=1e-12)


def test_split_count():
    assert oracle.split_count(0, 16, 8) == 0
    assert oracle.split_count(1, 16, 8) == 1
    assert oracle.split_count(33, 16, 2) == 2       # nb = 3, chunk = 2
    assert oracle.split_count(32768, 16, 32) == 32  # nb = 2048, chunk = 64
    assert oracle.split_count(17, 16, 32) == 2      # nb = 2, chunk = 1
    assert oracle.split_count(1000, 16, 1, 8) == 8  # nb = 63, fixed chunk 8


def test_combine_never_reads_past_the_valid_splits():
    c = _rand_case(23, B=2, lens=(40, 5))
    S = 8
    O, m, l = oracle.split_partials(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale, S)
    dense = _run(c)
    for s in range(c.B):
        n = oracle.split_count(int(c.context_lens[s]), c.BS, S)
        O[s, :, n:] = np.nan
        m[s, :, n:] = np.nan
        l[s, :, n:] = np.nan
    out = oracle.split_combine(O, m, l, c.context_lens, c.BS)
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------------------------------------------
# the append


def test_append_writes_rows_and_leaves_everything_else():
    rng = np.random.default_rng(31)
    N, Hkv, BS, D, T = 9, 3, 32, 64, 20
    k_pool = rng.standard_normal(W.k_pool_shape(N, Hkv, BS, D)).astype(np.float16)
    v_pool = rng.standard_normal(W.v_pool_shape(N, Hkv, BS, D)).astype(np.float16)
    k0, v0 = k_pool.copy(), v_pool.copy()
    slots = rng.choice(N * BS, size=T, replace=False).astype(np.int32)
    slots[3] = -1
    slots[7] = N * BS + 5  # outside the pool: skipped
    k = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float16)
    skipped = oracle.paged_kv_append(k, v, slots, k_pool, v_pool)
    assert skipped == 2
    touched = np.zeros((N, BS), bool)
    for i, sl in enumerate(slots):
        if 0 <= sl < N * BS:
            b, o = divmod(int(sl), BS)
            touched[b, o] = True
            for h in range(Hkv):
                assert np.array_equal(W.k_row(k_pool, b, h, o).view(np.uint16), k[i, h].view(np.uint16))
                assert np.array_equal(W.v_row(v_pool, b, h, o).view(np.uint16), v[i, h].view(np.uint16))
    for b in range(N):
        for o in range(BS):
            if not touched[b, o]:
                for h in range(Hkv):
                    assert np.array_equal(W.k_row(k_pool, b, h, o), W.k_row(k0, b, h, o))
                    assert np.array_equal(W.v_row(v_pool, b, h, o), W.v_row(v0, b, h, o))


def test_append_then_attention_sees_the_new_row():
    c = _rand_case(32, lens=(37, 16, 5), poison=True)
    # before the append the newest rows hold the poison value and the output is far off
    before = _run(c)
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, c.k_pool, c.v_pool)
    after = _run(c)
    for s in range(c.B):
        K, V = _rows(c, s, 0)
        assert np.array_equal(K[-1].astype(np.float16), c.k_new[s, 0])
    assert np.max(np.abs(before)) > 100 and np.max(np.abs(after)) < 10


# --------------------------------------------------------------------------------------------------------------
# paged varlen attention (several new rows per sequence, causal within them)


def _golden_varlen_cases():
    with open(os.path.join(GOLDEN, "varlen_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_varlen_cases(), ids=lambda c: c["name"])
def test_golden_varlen(case):
    k_pool, v_pool = _pools_from_rows(case)
    q = _pad32(case["q"], case["D"]).astype(np.float16)
    out = oracle.varlen_attention(q, k_pool, v_pool, case["block_tables"], case["cu_seqlens_q"],
                                  case["pos_offsets"], _num(case["scale"]), threads=2)
    np.testing.assert_allclose(out, _pad32(case["expected"], case["D"]), rtol=1e-14, atol=1e-14)


def _varlen(c, threads=4, units=None, k_pool=None, v_pool=None):
    return oracle.varlen_attention(c.q, c.k_pool if k_pool is None else k_pool, c.v_pool if v_pool is None else v_pool,
                                   c.block_tables, c.cu_seqlens_q, c.pos_offsets, c.scale, units=units, threads=threads)


def test_varlen_rows_are_decode_attention_at_their_position():
    # reduction to the decode oracle: row i of sequence s is decode attention of that query over pos + i + 1 rows
    c = W.build_varlen_case("v", 3, 8, 2, 64, 16, (3, 1, 6), (20, 0, 45), 31, poison_new=False)
    out = _varlen(c)
    for s in range(c.B):
        for i in range(int(c.q_lens[s])):
            t = int(c.cu_seqlens_q[s]) + i
            ref = oracle.decode_attention(c.q[t:t + 1], c.k_pool, c.v_pool, c.block_tables[s:s + 1],
                                          [int(c.pos_offsets[s]) + i + 1], c.scale, threads=1)
            assert np.array_equal(out[t], ref[0])


def test_varlen_matches_torch_causal_sdpa_on_gathered_rows():
    torch = pytest.importorskip("torch")
    for (Hq, Hkv, D, BS, ql, po) in [(8, 2, 64, 16, (4, 1, 7), (13, 0, 40)), (4, 4, 128, 32, (2, 9), (31, 64)),
                                     (16, 2, 64, 64, (5,), (70,))]:
        c = W.build_varlen_case("v", len(ql), Hq, Hkv, D, BS, ql, po, 100 + D + BS, poison_new=False)
        out = _varlen(c)
        for s in range(c.B):
            n_kv = int(c.final_lens[s])
            ks = np.empty((c.Hkv, n_kv, c.D))
            vs = np.empty((c.Hkv, n_kv, c.D))
            for t in range(n_kv):
                b = int(c.block_tables[s, t // c.BS])
                for h in range(c.Hkv):
                    ks[h, t] = W.k_row(c.k_pool, b, h, t % c.BS)
                    vs[h, t] = W.v_row(c.v_pool, b, h, t % c.BS)
            t0, t1 = int(c.cu_seqlens_q[s]), int(c.cu_seqlens_q[s + 1])
            qs = torch.from_numpy(c.q[t0:t1].astype(np.float64)).transpose(0, 1)        # [Hq][q_len][D]
            kk = torch.from_numpy(ks).repeat_interleave(c.G, dim=0)                      # [Hq][n_kv][D]
            vv = torch.from_numpy(vs).repeat_interleave(c.G, dim=0)
            allowed = torch.arange(n_kv)[None, :] <= (int(c.pos_offsets[s]) + torch.arange(t1 - t0))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qs, kk, vv, attn_mask=allowed, scale=c.scale)
            np.testing.assert_allclose(out[t0:t1], ref.transpose(0, 1).numpy(), rtol=1e-11, atol=1e-13)


def test_varlen_row_ignores_every_later_row():
    c = W.build_varlen_case("v", 2, 4, 2, 64, 16, (5, 3), (10, 29), 41, poison_new=False)
    out = _varlen(c)
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    # scramble every new row but the first of each sequence: each sequence's first new row must not move
    for s in range(c.B):
        for i in range(1, int(c.q_lens[s])):
            slot = int(c.slot_mapping[int(c.cu_seqlens_q[s]) + i])
            b, o = slot // c.BS, slot % c.BS
            W.set_k_row(kp, b, slice(None), o, np.full((c.Hkv, c.D), 7.0))
            W.set_v_row(vp, b, slice(None), o, np.full((c.Hkv, c.D), -9.0))
    out2 = _varlen(c, k_pool=kp, v_pool=vp)
    for s in range(c.B):
        t0 = int(c.cu_seqlens_q[s])
        assert np.array_equal(out[t0], out2[t0])
        assert not np.array_equal(out[t0 + 1], out2[t0 + 1])


def test_varlen_sequences_without_new_rows_and_units():
    c = W.build_varlen_case("v", 3, 4, 2, 64, 16, (2, 0, 3), (5, 9, 0), 43, poison_new=False)
    out = _varlen(c)
    assert out.shape == (5, 4, 64)
    units = np.array([[4, 3], [0, 1], [2, 0]], dtype=np.int32)
    part = _varlen(c, units=units)
    for j, (t, h) in enumerate(units):
        assert np.array_equal(part[j], out[t, h])


@pytest.mark.parametrize("cu,pos", [([1, 2, 3], [0, 0]), ([0, 2, 1], [0, 0]), ([0, 1, 3], [-1, 0]),
                                    ([0, 1, 3], [0, 47])])
def test_varlen_rejects_bad_prefix_sums_and_positions(cu, pos):
    c = W.build_varlen_case("v", 2, 4, 2, 64, 16, (1, 2), (3, 4), 44, poison_new=False, M=3)
    with pytest.raises(ValueError):
        oracle.varlen_attention(c.q, c.k_pool, c.v_pool, c.block_tables, cu, pos, c.scale)


# --------------------------------------------------------------------------------------------------------------
# sliding-window decode


def _golden_window_cases():
    with open(os.path.join(GOLDEN, "window_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_window_cases(), ids=lambda c: c["name"])
def test_golden_window(case):
    k_pool, v_pool = _pools_from_rows(case)
    q = _pad32(case["q"], case["D"]).astype(np.float16)
    out = oracle.decode_attention(q, k_pool, v_pool, case["block_tables"], case["context_lens"], _num(case["scale"]),
                                  threads=2, window=case["window"])
    np.testing.assert_allclose(out, _pad32(case["expected"], case["D"]), rtol=1e-14, atol=1e-14)


def test_window_at_least_the_context_is_plain_decode_and_one_row_returns_v():
    c = _rand_case(61, lens=(37, 16, 5))
    plain = _run(c)
    assert np.array_equal(oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale,
                                                  threads=4, window=37), plain)
    one = oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale, threads=4,
                                  window=1)
    for s in range(c.B):
        for hq in range(c.Hq):
            _, v = _rows(c, s, hq // c.G)
            assert np.array_equal(one[s, hq], v[-1])


def test_window_matches_torch_sdpa_over_the_last_rows():
    torch = pytest.importorskip("torch")
    for W_, lens, G, BS in [(5, (37, 16, 5, 2), 4, 16), (40, (100, 41, 39), 2, 32), (17, (64,), 1, 64)]:
        c = _rand_case(62 + W_, B=len(lens), Hq=4 * G, Hkv=4, BS=BS, lens=lens)
        out = oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale, threads=4,
                                      window=W_)
        for s in range(c.B):
            for hk in range(c.Hkv):
                ks, vs = _rows(c, s, hk)
                lo = max(0, len(ks) - W_)
                q = torch.from_numpy(c.q[s, hk * c.G:(hk + 1) * c.G].astype(np.float64))[:, None, :]
                kk = torch.from_numpy(ks[lo:])[None].expand(c.G, -1, -1)
                vv = torch.from_numpy(vs[lo:])[None].expand(c.G, -1, -1)
                ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=c.scale)[:, 0]
                np.testing.assert_allclose(out[s, hk * c.G:(hk + 1) * c.G], ref.numpy(), rtol=1e-11, atol=1e-13)


def test_window_ignores_rows_before_it():
    c = _rand_case(63, lens=(70, 33, 20))
    W_ = 20
    out = oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale, threads=4,
                                  window=W_)
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    for s in range(c.B):
        L = int(c.context_lens[s])
        for t in range(0, max(0, L - W_)):
            b = int(c.block_tables[s, t // c.BS])
            W.set_k_row(kp, b, slice(None), t % c.BS, np.full((c.Hkv, c.D), 30.0))
            W.set_v_row(vp, b, slice(None), t % c.BS, np.full((c.Hkv, c.D), -50.0))
    out2 = oracle.decode_attention(c.q, kp, vp, c.block_tables, c.context_lens, c.scale, threads=4, window=W_)
    assert np.array_equal(out, out2)
    assert not np.array_equal(_run(c), oracle.decode_attention(c.q, kp, vp, c.block_tables, c.context_lens, c.scale,
                                                               threads=4))


# --------------------------------------------------------------------------------------------------------------
# QKV-to-cache step: split QKV, q/k RMSNorm, RoPE, paged-cache write

def _golden_qkv_cases():
    with open(os.path.join(GOLDEN, "qkv_rope_hand.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_qkv_cases(), ids=lambda c: c["name"])
def test_golden_qkv(case):
    D, BS, N, Hkv = case["D"], case["BS"], case["N"], case["Hkv"]
    qkv = np.asarray(case["qkv"], dtype=np.float16)
    T = qkv.shape[0]
    qkv = np.ascontiguousarray(qkv.reshape(T, -1))
    k_pool, v_pool = _zero_pools(N, Hkv, BS, D)
    k_pool[...] = 0.25
    v_pool[...] = 0.25
    qw = None if case["q_norm_w"] is None else np.asarray(case["q_norm_w"], dtype=np.float16)
    kw = None if case["k_norm_w"] is None else np.asarray(case["k_norm_w"], dtype=np.float16)
    q, k, slots = oracle.qkv_norm_rope_paged(qkv, qw, kw, np.asarray(case["cos"], np.float32),
                                             np.asarray(case["sin"], np.float32), case["cu_seqlens_q"],
                                             case["rope_pos"], case["cache_pos"], case["block_tables"], k_pool,
                                             v_pool, case["eps"], case["qk_mode"])
    np.testing.assert_allclose(q, np.asarray(case["expected_q"], dtype=np.float64), rtol=0, atol=1e-6)
    np.testing.assert_allclose(k, np.asarray(case["expected_k"], dtype=np.float64), rtol=0, atol=1e-6)
    assert slots.tolist() == case["expected_slots"]
    ref = np.full_like(v_pool, 0.25)
    for r in case["expected_v_rows"]:
        W.set_v_row(ref, r["block"], r["head"], r["offset"], r["v"])
    assert np.array_equal(v_pool.view(np.uint16), ref.view(np.uint16))
    assert np.all(k_pool == np.float16(0.25)), "the oracle leaves k_pool to the caller"


def _qkv_small(seed=11, qk_mode=0, q_lens=(3, 1, 5), pos=(0, 17, 30), B=3, Hq=4, Hkv=2, D=64, BS=16, **kw):
    return W.build_qkv_case("small", B, Hq, Hkv, D, BS, list(q_lens), list(pos), seed, qk_mode=qk_mode, **kw)


def _qkv_run(c, cos=None, sin=None, qk_mode=None, v_pool=None):
    vc = c.varlen
    vp = vc.v_pool.copy() if v_pool is None else v_pool
    return oracle.qkv_norm_rope_paged(c.qkv, c.q_norm_w, c.k_norm_w, c.cos if cos is None else cos,
                                      c.sin if sin is None else sin, vc.cu_seqlens_q, vc.pos_offsets,
                                      vc.pos_offsets, vc.block_tables, vc.k_pool, vp, c.eps,
                                      c.qk_mode if qk_mode is None else qk_mode) + (vp,)


def _token_positions(vc):
    pos = np.empty(vc.T, dtype=np.int64)
    for s in range(vc.B):
        for i in range(int(vc.q_lens[s])):
            pos[vc.cu_seqlens_q[s] + i] = vc.pos_offsets[s] + i
    return pos


def _heads(c):
    vc = c.varlen
    return oracle.f16_to_f64(c.qkv).reshape(vc.T, vc.Hq + 2 * vc.Hkv, vc.D)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_qkv_rope_is_a_complex_rotation(D):
    """Without the norm, each head's dims j and j + D/2 form the complex number a + ib, which RoPE multiplies by
    cos + i sin of the token's table row (numpy complex arithmetic as the independent second opinion)."""
    c = _qkv_small(seed=21 + D, D=D, theta=1.0e4)
    vc = c.varlen
    q, k, _, _ = _qkv_run(c)
    x = _heads(c)
    half = D // 2
    z = x[..., :half] + 1j * x[..., half:]
    pos = _token_positions(vc)
    rot = (c.cos.astype(np.float64) + 1j * c.sin.astype(np.float64))[pos][:, None, :]
    want = z * rot
    got = np.concatenate([q, k], axis=1)
    np.testing.assert_allclose(got[..., :half], want.real[:, :vc.Hq + vc.Hkv], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., half:], want.imag[:, :vc.Hq + vc.Hkv], rtol=0, atol=1e-12)


def test_qkv_norm_is_torch_rms_norm():
    """With identity tables (cos 1, sin 0) the step is the RMS norm alone: torch's CPU rms_norm in float64, with the
    query weight on query heads and the key weight on key heads."""
    import torch
    import torch.nn.functional as F
    c = _qkv_small(seed=31, qk_mode=1, D=128, qkv_scale=3.0, eps=1e-3)
    vc = c.varlen
    ones, zeros = np.ones_like(c.cos), np.zeros_like(c.sin)
    q, k, _, _ = _qkv_run(c, cos=ones, sin=zeros)
    x = torch.from_numpy(_heads(c))
    qw = torch.from_numpy(oracle.f16_to_f64(c.q_norm_w))
    kw = torch.from_numpy(oracle.f16_to_f64(c.k_norm_w))
    eps = float(np.float32(c.eps))
    want_q = F.rms_norm(x[:, :vc.Hq], (vc.D,), qw, eps).numpy()
    want_k = F.rms_norm(x[:, vc.Hq:vc.Hq + vc.Hkv], (vc.D,), kw, eps).numpy()
    np.testing.assert_allclose(q, want_q, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(k, want_k, rtol=1e-13, atol=1e-13)


def test_qkv_position_zero_is_identity_and_pairs_keep_their_length():
    c = _qkv_small(seed=41, q_lens=(4, 2), pos=(0, 9), B=2, theta=1.0e4)
    vc = c.varlen
    q, k, _, _ = _qkv_run(c)
    x = _heads(c)
    # token 0 of sequence 0 sits at position 0: cos 1, sin 0 exactly
    assert np.array_equal(q[0], x[0, :vc.Hq]) and np.array_equal(k[0], x[0, vc.Hq:vc.Hq + vc.Hkv])
    half = vc.D // 2
    got = np.concatenate([q, k], axis=1)
    src = x[:, :vc.Hq + vc.Hkv]
    n_got = np.hypot(got[..., :half], got[..., half:])
    n_src = np.hypot(src[..., :half], src[..., half:])
    np.testing.assert_allclose(n_got, n_src, rtol=2e-7, atol=1e-12)  # float32 tables: cos^2 + sin^2 = 1 +- 1e-7


def test_qkv_scores_depend_only_on_relative_position():
    """RoPE's defining property: q at position p and k at p' give the score of q at p + d and k at p' + d.
    Sequence 1 repeats sequence 0's rows 37 positions later."""
    c = _qkv_small(seed=51, q_lens=(3, 3), pos=(2, 39), B=2, D=128, theta=1.0e4)
    vc = c.varlen
    c.qkv[3:6] = c.qkv[0:3]
    q, k, _, _ = _qkv_run(c)
    G = vc.Hq // vc.Hkv
    for i in range(3):
        for j in range(3):
            for hq in range(vc.Hq):
                a = q[i, hq] @ k[j, hq // G]
                b = q[3 + i, hq] @ k[3 + j, hq // G]
                scale = np.linalg.norm(q[i, hq]) * np.linalg.norm(k[j, hq // G])
                assert abs(a - b) <= 2e-6 * scale, (i, j, hq, a, b)


def test_qkv_value_rows_land_at_the_append_slots_and_nothing_else_changes():
    """The cache rows are the ones the paged append would use (the slot mapping the input generator derives from
    the tables); value rows are bit copies; every other pool element is untouched."""
    c = _qkv_small(seed=61, q_lens=(20, 1, 33), pos=(5, 16, 31), D=64, BS=32)
    vc = c.varlen
    before = vc.v_pool.copy()
    _, _, slots, vp = _qkv_run(c)
    assert np.array_equal(slots, vc.slot_mapping.astype(np.int64))
    x = c.qkv.reshape(vc.T, vc.Hq + 2 * vc.Hkv, vc.D)
    ref = before.copy()
    for t, slot in enumerate(vc.slot_mapping):
        W.set_v_row(ref, int(slot) // vc.BS, slice(None), int(slot) % vc.BS, x[t, vc.Hq + vc.Hkv:])
    assert np.array_equal(vp.view(np.uint16), ref.view(np.uint16))


def test_qkv_batched_call_equals_one_sequence_at_a_time():
    c = _qkv_small(seed=71, qk_mode=1, q_lens=(3, 0, 5), pos=(0, 7, 30))
    vc = c.varlen
    q, k, slots, vp = _qkv_run(c)
    vp1 = vc.v_pool.copy()
    for s in range(vc.B):
        a, b = int(vc.cu_seqlens_q[s]), int(vc.cu_seqlens_q[s + 1])
        q1, k1, sl1 = oracle.qkv_norm_rope_paged(np.ascontiguousarray(c.qkv[a:b]), c.q_norm_w, c.k_norm_w, c.cos,
                                                 c.sin, [0, b - a], vc.pos_offsets[s:s + 1],
                                                 vc.pos_offsets[s:s + 1], vc.block_tables[s:s + 1], vc.k_pool, vp1,
                                                 c.eps, c.qk_mode)
        assert np.array_equal(q1, q[a:b]) and np.array_equal(k1, k[a:b]) and np.array_equal(sl1, slots[a:b])
    assert np.array_equal(vp1.view(np.uint16), vp.view(np.uint16))


def test_qkv_rejects_bad_mode_positions_rows_and_tables():
    c = _qkv_small(seed=81)
    vc = c.varlen
    with pytest.raises(ValueError):
        _qkv_run(c, qk_mode=2)
    assert c.cos.shape[0] == 35  # the last token sits at position 34
    with pytest.raises(ValueError):
        _qkv_run(c, cos=c.cos[:34], sin=c.sin[:34])
    bad = vc.block_tables.copy()
    bad[2, 2] = -1
    with pytest.raises(ValueError):
        oracle.qkv_norm_rope_paged(c.qkv, c.q_norm_w, c.k_norm_w, c.cos, c.sin, vc.cu_seqlens_q, vc.pos_offsets,
                                   vc.pos_offsets, bad, vc.k_pool, vc.v_pool.copy(), c.eps, c.qk_mode)
    with pytest.raises(ValueError):  # cache rows past M * BS
        oracle.qkv_norm_rope_paged(c.qkv, c.q_norm_w, c.k_norm_w, c.cos, c.sin, vc.cu_seqlens_q, vc.pos_offsets,
                                   vc.pos_offsets + 64, vc.block_tables, vc.k_pool, vc.v_pool.copy(), c.eps,
                                   c.qk_mode)
    with pytest.raises(ValueError):
        oracle.qkv_norm_rope_paged(c.qkv, c.q_norm_w, c.k_norm_w, c.cos, c.sin, [0, 3, 2, 9], vc.pos_offsets,
                                   vc.pos_offsets, vc.block_tables, vc.k_pool, vc.v_pool.copy(), c.eps, c.qk_mode)
