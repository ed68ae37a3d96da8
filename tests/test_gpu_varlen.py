"""GPU parity of paged varlen attention (several new query rows per sequence, causal within them) against the
CPU oracle, through the C ABI: the new rows are appended with pkv_paged_kv_append, then attended; the oracle
applies the same append to its copy of the pools.  Bar: max|gpu - ref| <= 2e-3 and <= 1e-2 of max|ref|.
"""
import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import workloads as W
from test_gpu_parity import assert_close, say, torch_cuda, _dev  # noqa: F401  (fixture and helpers)

pytestmark = pytest.mark.gpu

# (Hq, Hkv, D, BS, new rows per sequence, positions of their first new row).  Tiles hold 16 / G new rows (two tiles
# per workgroup once a sequence has more than one), so these
# cover G = 4 (4 rows per tile, ragged tiles, a sequence without new rows, 16 rows = 4 tiles), G = 1 with D = 256
# (16 rows per tile), G = 16 (one row per tile), G = 3 (5 rows, 15 of 16 columns) and speculative-verify shapes.
VARLEN_GEOMS = [
    (8, 2, 64, 16, (1, 4, 7, 0, 16), (0, 30, 100, 12, 3)),
    (32, 8, 128, 16, (4, 4, 4, 4), (511, 1000, 63, 2040)),
    (16, 16, 256, 32, (3, 17), (40, 100)),
    (32, 2, 128, 64, (2, 5), (64, 130)),
    (12, 4, 128, 32, (5, 6), (20, 77)),
    (8, 8, 64, 16, (33,), (0,)),
]


def _run_case(torch, c, num_splits, max_q_len=0):
    from paged_kv_decode_04_amd import pkv
    kp, vp = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    pkv.paged_kv_append(_dev(torch, c.k_new), _dev(torch, c.v_new), _dev(torch, c.slot_mapping), kp, vp)
    out = pkv.paged_varlen_attention(_dev(torch, c.q), kp, vp, _dev(torch, c.block_tables),
                                     _dev(torch, c.cu_seqlens_q), _dev(torch, c.pos_offsets), c.scale,
                                     num_splits=num_splits, max_q_len=max_q_len)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _reference(c):
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, kp, vp)
    return oracle.varlen_attention(c.q, kp, vp, c.block_tables, c.cu_seqlens_q, c.pos_offsets, c.scale)


@pytest.mark.parametrize("geom", VARLEN_GEOMS, ids=lambda g: "Hq%d_Hkv%d_D%d_BS%d_T%d" % (g[:4] + (sum(g[4]),)))
@pytest.mark.parametrize("num_splits", [1, 3, 0])
def test_varlen_matches_oracle(torch_cuda, geom, num_splits):
    Hq, Hkv, D, BS, ql, po = geom
    c = W.build_varlen_case("varlen", len(ql), Hq, Hkv, D, BS, ql, po, 900 + D + BS + Hq)
    say("varlen %s S=%d" % (geom, num_splits))
    out = _run_case(torch_cuda, c, num_splits)
    assert_close(out, _reference(c), "varlen %s S=%d" % (geom, num_splits))


@pytest.mark.parametrize("max_q_len", [1, 5])
def test_varlen_small_grid_estimate_still_covers_every_row(torch_cuda, max_q_len):
    # max_q_len = 1 sizes the grid for one tile per sequence (4 rows at G = 4), 5 for one group of two tiles
    # (8 rows); the workgroups loop over the remaining tiles or groups
    c = W.build_varlen_case("varlen", 3, 8, 2, 128, 16, (9, 1, 14), (5, 200, 31), 951)
    ref = _reference(c)
    for S in (1, 2):
        out = _run_case(torch_cuda, c, S, max_q_len=max_q_len)
        assert_close(out, ref, "varlen max_q_len=%d S=%d" % (max_q_len, S))


def test_varlen_v2_full_size(torch_cuda):
    """Speculative verification with 8 new rows per sequence (two tiles of 4 rows sharing each K/V load), the
    bench workload at full size: 256 sampled (token, head) rows against the oracle."""
    c = W.config_v2()
    out = _run_case(torch_cuda, c, 0, max_q_len=8)
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, kp, vp)
    rng = np.random.default_rng(961)
    units = np.stack([rng.integers(0, c.T, 256), rng.integers(0, c.Hq, 256)], axis=1).astype(np.int32)
    units[:3] = [[0, 0], [c.T - 1, c.Hq - 1], [7, 5]]
    ref = oracle.varlen_attention(c.q, kp, vp, c.block_tables, c.cu_seqlens_q, c.pos_offsets, c.scale, units=units)
    assert_close(out[units[:, 0], units[:, 1]], ref, "v2 (8 new rows per sequence)")


def test_varlen_one_new_row_is_decode_attention(torch_cuda):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    lens = (300, 17, 1, 129)
    c = W.build_varlen_case("varlen", 4, 32, 8, 128, 16, (1, 1, 1, 1), tuple(L - 1 for L in lens), 952,
                            poison_new=False)
    out = _run_case(torch, c, 1)
    dec = pkv.paged_decode_attention(_dev(torch, c.q), _dev(torch, c.k_pool), _dev(torch, c.v_pool),
                                     _dev(torch, c.block_tables), _dev(torch, np.array(lens, np.int32)), c.scale,
                                     num_splits=1)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    assert_close(out, dec.astype(np.float64), "varlen q_len=1 vs decode")
    say("varlen q_len=1 bit-identical to decode: %s" % np.array_equal(out.view(np.uint16), dec.view(np.uint16)))


def test_varlen_empty_batch_is_a_no_op(torch_cuda):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    c = W.build_varlen_case("varlen", 2, 8, 2, 64, 16, (0, 0), (3, 9), 953)
    q = torch.zeros((0, 8, 64), dtype=torch.float16, device="cuda")
    out = pkv.paged_varlen_attention(q, _dev(torch, c.k_pool), _dev(torch, c.v_pool), _dev(torch, c.block_tables),
                                     _dev(torch, c.cu_seqlens_q), _dev(torch, c.pos_offsets), c.scale)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 64)


@pytest.mark.parametrize("num_splits", [1, 3])
def test_varlen_multi_round_grid_runs_longest_first(torch_cuda, num_splits):
    """80 sequences x 8 kv heads (more than one round of the CUs): the sequences run longest first through order
    records in the library workspace; every output against the oracle.  Lengths include empty sequences and ties."""
    rng = np.random.default_rng(971)
    ql = rng.integers(0, 10, 80)
    ql[[2, 9]] = 0
    po = rng.integers(0, 500, 80)
    po[[4, 5]] = 300
    ql[[4, 5]] = 3  # equal keys
    c = W.build_varlen_case("varlen", 80, 32, 8, 128, 16, ql, po, 972)
    say("varlen multi-round S=%d" % num_splits)
    out = _run_case(torch_cuda, c, num_splits, max_q_len=int(ql.max()))
    assert_close(out, _reference(c), "varlen multi-round S=%d" % num_splits)


def test_varlen_capture_of_a_multi_round_grid_needs_no_warm_up(torch_cuda):
    """Captured on a stream no call has used, a multi-round varlen grid keeps id order rather than growing the
    library workspace under capture; its replays match the eager result bit for bit."""
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    rng = np.random.default_rng(973)
    c = W.build_varlen_case("varlen", 48, 32, 8, 128, 16, rng.integers(1, 5, 48), rng.integers(0, 400, 48), 974,
                            poison_new=False)
    q, kp, vp = _dev(torch, c.q), _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    bt, cu, pos = _dev(torch, c.block_tables), _dev(torch, c.cu_seqlens_q), _dev(torch, c.pos_offsets)
    out = torch.empty_like(q)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pkv.paged_varlen_attention(q, kp, vp, bt, cu, pos, c.scale, out=out, num_splits=1, max_q_len=4)
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
        torch.cuda.synchronize()
    eager = pkv.paged_varlen_attention(q, kp, vp, bt, cu, pos, c.scale, num_splits=1, max_q_len=4)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), eager.view(torch.int16))
    ref = oracle.varlen_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.cu_seqlens_q, c.pos_offsets, c.scale)
    assert_close(eager.cpu().numpy(), ref, "varlen eager, longest first")
