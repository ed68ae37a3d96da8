"""Seeded random sweep over geometries (head dim, block size, kv heads, group size, batch, lengths) and entry points:
decode attention at one pass, automatic and forced splits; the decode step (pools bit-exact); the sliding window;
varlen attention and the varlen step.  Every draw is checked against the CPU oracle at the usual bar
(max|err| <= 2e-3 and <= 1e-2 of max|ref|), so combinations no hand-picked case names are covered too.
"""
import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import workloads as W
from test_gpu_parity import assert_close, say, torch_cuda, _dev, _upload, full_new_rows  # noqa: F401

pytestmark = pytest.mark.gpu

DRAWS = 24


def _geometry(rng):
    D = int(rng.choice([64, 128, 256]))
    BS = int(rng.choice([16, 32, 64]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    B = int(rng.integers(1, 7))
    return D, BS, Hkv, G, B


@pytest.mark.parametrize("draw", range(DRAWS))
def test_decode_entry_points_on_random_geometries(torch_cuda, draw):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    rng = np.random.default_rng(20000 + draw)
    D, BS, Hkv, G, B = _geometry(rng)
    lens = rng.integers(0, 400, B)
    lens[rng.integers(0, B)] = max(1, int(lens.max()))
    what = "draw %d: D=%d BS=%d Hkv=%d G=%d lens=%s" % (draw, D, BS, Hkv, G, lens.tolist())
    say(what)
    c = W.small_case(20100 + draw, B, G * Hkv, Hkv, D, BS, lens, poison=True, extra_blocks=2)
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, kp, vp)
    ref = oracle.decode_attention(c.q, kp, vp, c.block_tables, c.context_lens, c.scale)
    # the decode step (append + attention) on the poisoned pools
    kn, vn = full_new_rows(c)
    dk, dv = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    S = int(rng.integers(2, 7))
    for splits in (1, 0, S):
        dk.copy_(_dev(torch, c.k_pool))
        dv.copy_(_dev(torch, c.v_pool))
        out = pkv.paged_decode_step(_dev(torch, c.q), _dev(torch, kn), _dev(torch, vn), dk, dv,
                                    _dev(torch, c.block_tables), _dev(torch, c.context_lens), c.scale,
                                    num_splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(dk.cpu().numpy().view(np.uint16), kp.view(np.uint16)), what
        assert np.array_equal(dv.cpu().numpy().view(np.uint16), vp.view(np.uint16)), what
        assert_close(out.cpu().numpy(), ref, "%s step S=%d" % (what, splits))
    # attention alone and the sliding window, over the appended pools
    d = dict(q=_dev(torch, c.q), kp=_dev(torch, kp), vp=_dev(torch, vp), bt=_dev(torch, c.block_tables),
             cl=_dev(torch, c.context_lens))
    out = pkv.paged_decode_attention(d["q"], d["kp"], d["vp"], d["bt"], d["cl"], c.scale, num_splits=S)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "%s attention S=%d" % (what, S))
    window = int(rng.integers(1, 300))
    refw = oracle.decode_attention(c.q, kp, vp, c.block_tables, c.context_lens, c.scale, window=window)
    for splits in (1, S):
        out = pkv.paged_decode_attention_window(d["q"], d["kp"], d["vp"], d["bt"], d["cl"], c.scale, window,
                                                num_splits=splits)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), refw, "%s window %d S=%d" % (what, window, splits))


@pytest.mark.parametrize("draw", range(DRAWS))
def test_varlen_entry_points_on_random_geometries(torch_cuda, draw):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    rng = np.random.default_rng(21000 + draw)
    D, BS, Hkv, G, B = _geometry(rng)
    ql = rng.integers(0, 12, B)
    ql[rng.integers(0, B)] = max(1, int(ql.max()))
    po = rng.integers(0, 300, B)
    what = "draw %d: D=%d BS=%d Hkv=%d G=%d q_lens=%s pos=%s" % (draw, D, BS, Hkv, G, ql.tolist(), po.tolist())
    say(what)
    c = W.build_varlen_case("sweep", B, G * Hkv, Hkv, D, BS, ql, po, 21100 + draw)
    kp, vp = c.k_pool.copy(), c.v_pool.copy()
    oracle.paged_kv_append(c.k_new, c.v_new, c.slot_mapping, kp, vp)
    ref = oracle.varlen_attention(c.q, kp, vp, c.block_tables, c.cu_seqlens_q, c.pos_offsets, c.scale)
    qmax = int(ql.max())
    for splits in (1, int(rng.integers(2, 5))):
        dk, dv = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
        out = pkv.paged_varlen_step(_dev(torch, c.q), _dev(torch, c.k_new), _dev(torch, c.v_new), dk, dv,
                                    _dev(torch, c.block_tables), _dev(torch, c.cu_seqlens_q),
                                    _dev(torch, c.pos_offsets), c.scale, qmax, num_splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(dk.cpu().numpy().view(np.uint16), kp.view(np.uint16)), what
        assert np.array_equal(dv.cpu().numpy().view(np.uint16), vp.view(np.uint16)), what
        assert_close(out.cpu().numpy(), ref, "%s varlen step S=%d" % (what, splits))
        out = pkv.paged_varlen_attention(_dev(torch, c.q), _dev(torch, kp), _dev(torch, vp),
                                         _dev(torch, c.block_tables), _dev(torch, c.cu_seqlens_q),
                                         _dev(torch, c.pos_offsets), c.scale, num_splits=splits,
                                         max_q_len=int(rng.integers(1, qmax + 1)))
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, "%s varlen attention S=%d" % (what, splits))
