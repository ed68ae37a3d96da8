"""Ordered single passes whose longest sequences are split into pieces: a grid of several rounds of the CUs in
which a sequence needs more rows than a CU's fair share of the launch (all rows times the kv heads over the CUs).
The ordering launch gives such a sequence several records, each piece runs as a tile of its own, and the last
piece of each (sequence, kv head) to finish merges the pieces' partials in piece order.

Checked here: the outputs against the oracle (the same bar as every attention test), the same bits on every call
and on graph replays (the merge order does not depend on which piece ends last), the decode step through the
append launch that writes the records, and -- on the CPU, by a mirror of the rule -- that each case does split.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import workloads as W

ATOL = 2e-3
RTOL_MAX = 1e-2
MIN_PIECE_ROWS = 1024


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def pieces_of(lens, Hkv, cus, cap_rows):
    """The piece count of every sequence under the rule (mirrored on the host for the tests only)."""
    keys = np.clip(np.asarray(lens, dtype=np.int64), 0, cap_rows)
    fair = -(-int(keys.sum()) * Hkv // cus)
    C = max(MIN_PIECE_ROWS, -(-fair // 64) * 64)
    out = []
    for k in keys:
        if k <= C:
            out.append(1)
            continue
        n = -(-int(k) // C)
        pr = -(-(-(-int(k) // n)) // 64) * 64
        out.append(-(-int(k) // pr))
    return np.array(out)


# (seed, B, Hq, Hkv, D, BS, lens): a few long sequences among short ones; B * Hkv > 256 workgroups
def _lens(seed, B, long_rows, lo, hi):
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, B).astype(np.int32)
    lens[[1, 7, 20][:len(long_rows)]] = long_rows
    return lens


CASES = [
    (601, 64, 32, 8, 128, 16, _lens(601, 64, [12000, 5000, 1025], 40, 400)),
    (602, 48, 16, 16, 256, 32, _lens(602, 48, [9000], 30, 300)),
    (603, 40, 64, 8, 64, 64, _lens(603, 40, [7000, 2500], 20, 200)),
]


def test_the_cases_split_under_the_rule():
    """CPU: on a 256-CU device every case has a sequence in several pieces, and fewer extra records than
    256 / Hkv (the grid's room for them)."""
    for seed, B, Hq, Hkv, D, BS, lens in CASES:
        n = pieces_of(lens, Hkv, 256, 1 << 30)
        assert n.max() > 1 and (n - 1).sum() < 256 / Hkv, (seed, n.max(), (n - 1).sum())
    # the boundary: a key of exactly C rows stays whole, C + 1 rows make two pieces
    n = pieces_of([1024, 1025] + [10] * 62, 8, 256, 1 << 30)
    assert n[0] == 1 and n[1] == 2


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_decode_04_amd import pkv
    pkv.load()  # raises if the HIP library is missing: no fallback
    return torch


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def assert_close(gpu, ref, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    top = float(np.max(np.abs(ref))) if ref.size else 0.0
    worst = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(gpu)), "%s: non-finite output" % what
    say("%s: max|err| %.3e, max|ref| %.3e" % (what, worst, top))
    assert worst <= ATOL, "%s: max|err| %.3e > %.1e" % (what, worst, ATOL)
    assert worst <= RTOL_MAX * max(top, 1e-30) or worst == 0.0, "%s: relative %.3e" % (what, worst / top)


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Hkv%d_D%d_BS%d" % (c[1], c[3], c[4], c[5]))
def test_pieces_match_the_oracle_and_repeat_exactly(torch_cuda, case):
    torch = torch_cuda
    from paged_kv_decode_04_amd import pkv
    seed, B, Hq, Hkv, D, BS, lens = case
    c = W.small_case(seed, B, Hq, Hkv, D, BS, lens)
    n = pieces_of(lens, Hkv, pkv.device_cu_count(), c.M * BS)
    say("pieces B=%d Hkv=%d D=%d BS=%d: longest %d rows in %d pieces, %d extra records" %
        (B, Hkv, D, BS, int(lens.max()), int(n.max()), int((n - 1).sum())))
    assert n.max() > 1
    d = [_dev(torch, x) for x in (c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens)]
    outs = []
    for _ in range(3):
        outs.append(pkv.paged_decode_attention(*d, c.scale).cpu().numpy())
    ref = oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    assert_close(outs[0], ref, "pieces B=%d D=%d" % (B, D))
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint16), outs[0].view(np.uint16))
    # the same call through a caller workspace runs whole sequences in id order: within the bar of it
    plan = pkv.plan_decode(c.B, c.Hq, c.Hkv, c.D, c.BS, c.M)
    ws = torch.empty(max(256, plan["workspace_bytes"]), dtype=torch.uint8, device="cuda")
    plain = pkv.paged_decode_attention(*d, c.scale, workspace=ws).cpu().numpy()
    assert np.max(np.abs(plain.astype(np.float64) - outs[0].astype(np.float64))) <= ATOL


@pytest.mark.gpu
def test_pieces_in_the_decode_step(torch_cuda):
    """The decode step of a multi-round grid: the append launch writes the new rows and the piece records, then the
    ordered attention -- the pools bit-exact and the output within the bar, against the oracle's append then
    attention."""
    torch = torch_cuda
    from paged_kv_decode_04_amd import pkv
    seed, B, Hq, Hkv, D, BS, lens = CASES[0]
    c = W.small_case(seed + 50, B, Hq, Hkv, D, BS, lens, poison=True, extra_blocks=4)
    nz = np.nonzero(c.context_lens > 0)[0]
    kn = np.zeros((c.B, c.Hkv, c.D), np.float16)
    vn = np.zeros_like(kn)
    kn[nz], vn[nz] = c.k_new, c.v_new
    dk, dv = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    out = pkv.paged_decode_step(_dev(torch, c.q), _dev(torch, kn), _dev(torch, vn), dk, dv,
                                _dev(torch, c.block_tables), _dev(torch, c.context_lens), c.scale)
    torch.cuda.synchronize()
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, kp, vp)
    assert np.array_equal(dk.cpu().numpy().view(np.uint16), kp.view(np.uint16))
    assert np.array_equal(dv.cpu().numpy().view(np.uint16), vp.view(np.uint16))
    ref = oracle.decode_attention(c.q, kp, vp, c.block_tables, c.context_lens, c.scale)
    assert_close(out.cpu().numpy(), ref, "decode step with pieces")


@pytest.mark.gpu
def test_pieces_under_graph_replay(torch_cuda):
    """A captured ordered attention call replayed while the device-resident lengths change (the longest sequence
    grows past a piece boundary): every replay bit-identical to the eager call on the same state."""
    torch = torch_cuda
    from paged_kv_decode_04_amd import pkv
    seed, B, Hq, Hkv, D, BS, lens = CASES[0]
    grown = lens.copy()
    grown[1] += 1500
    c = W.small_case(seed + 70, B, Hq, Hkv, D, BS, grown)  # the tables hold the grown sequence
    q, kp, vp, bt = (_dev(torch, x) for x in (c.q, c.k_pool, c.v_pool, c.block_tables))
    cl_g, cl_e = _dev(torch, lens), _dev(torch, lens)
    out_g = torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")
    out_e = torch.empty_like(out_g)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        pkv.paged_decode_attention(q, kp, vp, bt, cl_g, c.scale, out=out_g)  # sizes the stream's workspace
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pkv.paged_decode_attention(q, kp, vp, bt, cl_g, c.scale, out=out_g)
    torch.cuda.synchronize()
    for i, extra in enumerate((0, 700, 1500)):
        cur = lens.copy()
        cur[1] += extra
        cl_g.copy_(torch.from_numpy(cur))
        cl_e.copy_(torch.from_numpy(cur))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        pkv.paged_decode_attention(q, kp, vp, bt, cl_e, c.scale, out=out_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), "replay %d" % i
        say("pieces graph replay %d (longest %d rows): bit-identical to the eager call" % (i, int(cur.max())))
    ref = oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, cur, c.scale)
    assert_close(out_g.cpu().numpy(), ref, "pieces graph last replay")
