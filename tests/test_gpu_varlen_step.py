"""GPU parity of the varlen step (pkv_paged_varlen_step: each sequence's new K/V rows written through its block table
at rows pos .. pos + q_len - 1, then varlen attention over the updated pools) against the oracle's append followed
by its varlen attention, through the C ABI.  Both launch forms are covered: one launch whose workgroups write the new
rows themselves (a single pass, at most 32 new rows per sequence, no more workgroups than CUs, one tile per group at
head dim 256), and the append launch then attention (splits, more rows, larger grids).
Bar: pools bit-exact; attention max|gpu - ref| <= 2e-3 and <= 1e-2 of max|ref|; the step's output bit-identical to
pkv_paged_kv_append followed by pkv_paged_varlen_attention with the same split count.
"""
import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import workloads as W
from test_gpu_parity import assert_close, say, torch_cuda, _dev  # noqa: F401  (fixture and helpers)

pytestmark = pytest.mark.gpu

# (Hq, Hkv, D, BS, new rows per sequence, position of each sequence's first new row)
STEP_GEOMS = [
    (8, 2, 64, 16, (1, 4, 7, 0, 16), (0, 30, 100, 12, 3)),  # G=4: ragged tiles, no rows, two tiles per group
    (32, 8, 128, 16, (4, 4, 4, 4), (511, 1000, 63, 2040)),  # speculative-verify shape, rows crossing units
    (32, 8, 128, 16, (32, 17, 1), (15, 0, 47)),  # 32 rows from row 15: three 16-row units, four blocks
    (12, 4, 128, 32, (5, 6), (20, 77)),  # G=3: 15 of 16 columns
    (32, 2, 128, 64, (2, 5), (64, 130)),  # G=16: one row per tile
    (16, 16, 256, 32, (3, 9), (40, 100)),  # head dim 256, one tile per sequence (one launch)
    (16, 16, 256, 32, (3, 17), (40, 100)),  # head dim 256, two tiles per group (append launch, then attention)
    (8, 8, 64, 16, (33,), (0,)),  # more than 32 new rows (append launch, then attention)
]


def _reference(c):
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, kp, vp)
    return kp, vp, oracle.varlen_attention(c.q, kp, vp, c.block_tables, c.cu_seqlens_q, c.pos_offsets, c.scale)


def _step(torch, c, num_splits, max_q_len):
    from paged_kv_decode_04_amd import pkv
    kp, vp = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    out = pkv.paged_varlen_step(_dev(torch, c.q), _dev(torch, c.k_new), _dev(torch, c.v_new), kp, vp,
                                _dev(torch, c.block_tables), _dev(torch, c.cu_seqlens_q), _dev(torch, c.pos_offsets),
                                c.scale, max_q_len, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), kp.cpu().numpy(), vp.cpu().numpy()


def _two_calls(torch, c, num_splits, max_q_len):
    from paged_kv_decode_04_amd import pkv
    kp, vp = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    pkv.paged_kv_append(_dev(torch, c.k_new), _dev(torch, c.v_new), _dev(torch, c.slot_mapping), kp, vp)
    out = pkv.paged_varlen_attention(_dev(torch, c.q), kp, vp, _dev(torch, c.block_tables),
                                     _dev(torch, c.cu_seqlens_q), _dev(torch, c.pos_offsets), c.scale,
                                     num_splits=num_splits, max_q_len=max_q_len)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _assert_pools(kp, vp, rk, rv, what):
    assert np.array_equal(kp.view(np.uint16), rk.view(np.uint16)), "%s: K pool differs from the oracle's" % what
    assert np.array_equal(vp.view(np.uint16), rv.view(np.uint16)), "%s: V pool differs from the oracle's" % what


@pytest.mark.parametrize("geom", STEP_GEOMS, ids=lambda g: "Hq%d_Hkv%d_D%d_BS%d_T%d" % (g[:4] + (sum(g[4]),)))
@pytest.mark.parametrize("num_splits", [1, 3])
def test_varlen_step_matches_oracle(torch_cuda, geom, num_splits):
    Hq, Hkv, D, BS, ql, po = geom
    c = W.build_varlen_case("step", len(ql), Hq, Hkv, D, BS, ql, po, 1300 + D + BS + Hq + sum(ql))
    what = "varlen step %s S=%d" % (geom, num_splits)
    say(what)
    out, kp, vp = _step(torch_cuda, c, num_splits, max(ql))
    rk, rv, ref = _reference(c)
    _assert_pools(kp, vp, rk, rv, what)
    assert_close(out, ref, what)
    two = _two_calls(torch_cuda, c, num_splits, max(ql))
    assert np.array_equal(out.view(np.uint16), two.view(np.uint16)), "%s: differs from append + attention" % what


@pytest.mark.parametrize("geom", [(40, 32, 8, 128, 16, 6), (40, 16, 16, 256, 32, 3), (160, 8, 2, 64, 64, 21)],
                         ids=lambda g: "B%d_Hq%d_Hkv%d_D%d_BS%d_q%d" % g)
def test_varlen_step_grid_past_the_cus_takes_two_launches(torch_cuda, geom):
    """More workgroups than CUs: the append launch (whole panels, its extra workgroups writing the dispatch-order
    records), then attention longest first.  Pools bit-exact, output against the oracle and bit-identical to the
    slot-mapping append followed by varlen attention (whose order comes from a launch of its own)."""
    B, Hq, Hkv, D, BS, qmax = geom
    rng = np.random.default_rng(1351 + B + D)
    ql = rng.integers(0, qmax, B)
    ql[0] = qmax - 1
    po = rng.integers(0, 300, B)
    c = W.build_varlen_case("step", B, Hq, Hkv, D, BS, ql, po, 1352 + D)
    what = "step %s" % (geom,)
    say(what)
    out, kp, vp = _step(torch_cuda, c, 0, int(ql.max()))
    rk, rv, ref = _reference(c)
    _assert_pools(kp, vp, rk, rv, what)
    assert_close(out, ref, what)
    two = _two_calls(torch_cuda, c, 0, int(ql.max()))
    assert np.array_equal(out.view(np.uint16), two.view(np.uint16)), "%s: differs from append + attention" % what


def test_varlen_step_rows_of_a_missing_block_are_not_written(torch_cuda):
    # sequence 1's second block (rows 16..31, holding its new rows 16..19) names no pool block: nothing is written
    # there and those rows are masked; the other sequence is unaffected
    c = W.build_varlen_case("step", 2, 8, 2, 64, 16, (4, 4), (30, 16), 1361)
    c.block_tables[1, 1] = c.N + 5
    out, kp, vp = _step(torch_cuda, c, 1, 4)
    rk, rv = c.k_pool.copy(), c.v_pool.copy()
    slots = c.slot_mapping.copy()
    slots[4:] = -1  # the oracle appends sequence 0's rows only
    oracle.paged_kv_append(c.k_new, c.v_new, slots, rk, rv)
    _assert_pools(kp, vp, rk, rv, "missing block")
    ref0 = oracle.varlen_attention(c.q[:4], rk, rv, c.block_tables[:1], c.cu_seqlens_q[:2], c.pos_offsets[:1],
                                   c.scale)
    assert_close(out[:4], ref0, "missing block: the intact sequence")


@pytest.mark.parametrize("name", ["v1", "v2", "v3"])
def test_varlen_step_full_size(torch_cuda, name):
    """The step on the bench's v1 / v2 workloads (32 sequences, 4 or 8 new rows each, one launch) and v3 (256
    sequences of mixed lengths, 2048 workgroups: the append launch, the dispatch order, then attention longest first):
    pools bit-exact and 256 sampled (token, head) rows against the oracle."""
    c = W.VARLEN_CONFIGS[name]()
    say("varlen step %s full size" % name)
    out, kp, vp = _step(torch_cuda, c, 0, int(c.q_lens.max()))
    rk, rv = c.k_pool.copy(), c.v_pool.copy()
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, rk, rv)
    _assert_pools(kp, vp, rk, rv, "%s step" % name)
    rng = np.random.default_rng(1371)
    units = np.stack([rng.integers(0, c.T, 256), rng.integers(0, c.Hq, 256)], axis=1).astype(np.int32)
    units[:3] = [[0, 0], [c.T - 1, c.Hq - 1], [7, 5]]
    ref = oracle.varlen_attention(c.q, rk, rv, c.block_tables, c.cu_seqlens_q, c.pos_offsets, c.scale, units=units)
    assert_close(out[units[:, 0], units[:, 1]], ref, "%s step" % name)


@pytest.mark.parametrize("num_splits", [1, 2])
def test_varlen_step_with_a_loose_max_q_len(torch_cuda, num_splits):
    """max_q_len far above every sequence's new rows (40 against at most 5, the append launch then has idle unit
    slots; rows spanning two 16-row units and a block boundary): pools bit-exact, output against the oracle."""
    c = W.build_varlen_case("step", 5, 16, 4, 64, 32, (5, 0, 3, 4, 1), (14, 9, 30, 0, 63), 1381)
    what = "loose max_q_len S=%d" % num_splits
    say(what)
    out, kp, vp = _step(torch_cuda, c, num_splits, 40)
    rk, rv, ref = _reference(c)
    _assert_pools(kp, vp, rk, rv, what)
    assert_close(out, ref, what)
