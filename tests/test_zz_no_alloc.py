"""pkv_paged_decode_attention_noalloc: decode attention for callers that cannot allocate, its split-K partials and
dispatch-order records in the library's fixed device scratch.  Checked through the C ABI against
pkv_paged_decode_attention (the same kernels and plan, so bit-identical output) and against the oracle, on two calls
in a row with the second one smaller, on a grid of several rounds (records in the scratch), on a graph captured on a
stream no call has warmed up, and for a plan larger than the scratch (a clean PKV_EWORKSPACE)."""
import os
import re

import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import pkv
from paged_kv_decode_04_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ATOL = 2e-3


def _say(*a):
    print("[no-alloc]", *a, flush=True)


def test_scratch_limit_matches_the_header():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        m = re.search(r"#define PKV_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and (int(m.group(1)) << int(m.group(2))) == pkv.NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load()
    return torch


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _upload(torch, c):
    return [_dev(torch, x) for x in (c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens)]


def _against_both(torch, c, num_splits, what):
    """One no-allocation call against pkv_paged_decode_attention (bit-identical) and the oracle."""
    q, kp, vp, bt, cl = _upload(torch, c)
    out = torch.full_like(q, float("nan"))
    pkv.paged_decode_attention_noalloc(q, kp, vp, bt, cl, c.scale, out, num_splits=num_splits)
    ref_call = pkv.paged_decode_attention(q, kp, vp, bt, cl, c.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_call.view(torch.int16)), what
    ref = oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    err = float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref)))
    _say("%s: bit-identical to pkv_paged_decode_attention, max|err| vs oracle %.3e" % (what, err))
    assert err <= ATOL and err <= 1e-2 * float(np.max(np.abs(ref)))


@pytest.mark.gpu
@pytest.mark.parametrize("num_splits", [0, 5])
def test_two_calls_in_a_row_the_second_smaller(torch_cuda, num_splits):
    torch = torch_cuda
    big = W.small_case(901 + num_splits, 24, 32, 8, 128, 16, tuple(100 + (389 * i) % 2900 for i in range(24)))
    small = W.small_case(902 + num_splits, 3, 8, 2, 64, 16, (700, 33, 260))
    _against_both(torch, big, num_splits, "first call, 24 sequences, num_splits=%d" % num_splits)
    _against_both(torch, small, num_splits, "second call, 3 sequences, num_splits=%d" % num_splits)


@pytest.mark.gpu
def test_multi_round_grid_keeps_its_order_records_in_the_scratch(torch_cuda):
    """64 x 8 workgroups (more than one round of the CUs): the longest-first records go to the scratch; then a
    smaller split call reuses the same scratch."""
    torch = torch_cuda
    lens = tuple(1 + (211 * i) % 1500 for i in range(64))
    _against_both(torch, W.small_case(911, 64, 32, 8, 128, 16, lens), 1, "64 sequences, single pass")
    _against_both(torch, W.small_case(912, 6, 32, 8, 128, 16, (900, 4, 1200, 17, 640, 333)), 4,
                  "then 6 sequences, 4 splits")


@pytest.mark.gpu
def test_capture_on_a_fresh_stream(torch_cuda):
    """Captured on a stream no call has used (the library-workspace call would need to allocate there); replays
    with eager work and synchronisations between them match the eager call bit for bit."""
    torch = torch_cuda
    c = W.small_case(921, 5, 32, 8, 128, 16, (1500, 70, 800, 2047, 300))
    q, kp, vp, bt, cl = _upload(torch, c)
    out = torch.empty_like(q)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pkv.paged_decode_attention_noalloc(q, kp, vp, bt, cl, c.scale, out, num_splits=6)
    torch.cuda.synchronize()
    eager = torch.empty_like(q)
    pkv.paged_decode_attention_noalloc(q, kp, vp, bt, cl, c.scale, eager, num_splits=6)
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), "replay %d" % i
        _say("replay %d bit-identical to the eager call" % i)


@pytest.mark.gpu
def test_a_plan_beyond_the_scratch_is_refused(torch_cuda):
    torch = torch_cuda
    B, Hq, Hkv, D, BS = 512, 64, 8, 128, 16
    q = torch.zeros((B, Hq, D), dtype=torch.float16, device="cuda")
    kp = torch.zeros(W.k_pool_shape(1, Hkv, BS, D), dtype=torch.float16, device="cuda")
    vp = torch.zeros(W.v_pool_shape(1, Hkv, BS, D), dtype=torch.float16, device="cuda")
    bt = torch.zeros((B, 4), dtype=torch.int32, device="cuda")
    cl = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    need = pkv.decode_workspace_bytes(B, Hq, D, 16)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_decode_attention_noalloc(q, kp, vp, bt, cl, 0.1, out, num_splits=16)
    assert e.value.code == pkv.PKV_EWORKSPACE
    assert "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
