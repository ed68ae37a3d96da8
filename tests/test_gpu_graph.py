"""Graph-replayable decode: a decode step captured once in a HIP graph (torch.cuda.graph) replays correctly while
the device-resident state moves on -- the context lengths grow by one each step, new q and new K/V rows (or new QKV
rows) arrive -- with the program's own eager work and synchronisations between replays.  Every replay is checked bit
for bit against the same step run eagerly on a separate copy of the state, and the last one against the oracle run
on a state the oracle evolved itself over the same steps.
"""
import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import workloads as W
from test_gpu_parity import assert_close, say, torch_cuda, _dev  # noqa: F401  (fixture and helpers)

pytestmark = pytest.mark.gpu

STEPS = 5


def _state(torch, c, lens0):
    return dict(q=_dev(torch, c.q), kn=torch.zeros((c.B, c.Hkv, c.D), dtype=torch.float16, device="cuda"),
                vn=torch.zeros((c.B, c.Hkv, c.D), dtype=torch.float16, device="cuda"),
                kp=_dev(torch, c.k_pool), vp=_dev(torch, c.v_pool), bt=_dev(torch, c.block_tables),
                cl=_dev(torch, lens0), out=torch.empty((c.B, c.Hq, c.D), dtype=torch.float16, device="cuda"))


@pytest.mark.parametrize("B", [4, 40])
@pytest.mark.parametrize("num_splits", [1, 3])
def test_decode_step_graph_replays_follow_device_state(torch_cuda, num_splits, B):
    """B = 4: one launch per step; B = 40 (320 workgroups, more than one round of the CUs): the append launch,
    which also ranks the sequences longest first, then the ordered attention -- the order recomputed from the
    device-resident lengths on every replay."""
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    lens0 = (np.array([100, 31, 47, 16], dtype=np.int32) if B == 4 else
             np.random.default_rng(810).integers(1, 300, B).astype(np.int32))
    c = W.small_case(811 + num_splits + B, B, 32, 8, 128, 16, lens0 + STEPS)  # tables hold the grown sequences
    rng = np.random.default_rng(812)
    g_state, e_state = _state(torch, c, lens0), _state(torch, c, lens0)

    def step(st):
        pkv.paged_decode_step(st["q"], st["kn"], st["vn"], st["kp"], st["vp"], st["bt"], st["cl"], c.scale,
                              st["out"], num_splits=num_splits)

    stream = torch.cuda.Stream()
    warm = _state(torch, c, lens0)
    with torch.cuda.stream(stream):
        step(warm)  # sizes this stream's workspace before capture
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(g_state)
    torch.cuda.synchronize()
    # capture records work without running it: restore the state a first replay must start from
    for k in ("kp", "vp", "out"):
        g_state[k].copy_(e_state[k])
    kp_o, vp_o = c.k_pool.copy(), c.v_pool.copy()  # the oracle's own pools, advanced by the oracle's append
    lens = lens0.copy()
    for i in range(STEPS):
        q = rng.standard_normal((c.B, c.Hq, c.D)).astype(np.float16)
        kn = rng.standard_normal((c.B, c.Hkv, c.D)).astype(np.float16)
        vn = rng.standard_normal((c.B, c.Hkv, c.D)).astype(np.float16)
        for st in (g_state, e_state):
            st["cl"].add_(1)
            st["q"].copy_(torch.from_numpy(q))
            st["kn"].copy_(torch.from_numpy(kn))
            st["vn"].copy_(torch.from_numpy(vn))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e_state)
        torch.cuda.synchronize()
        for k in ("out", "kp", "vp"):
            assert torch.equal(g_state[k].view(torch.int16), e_state[k].view(torch.int16)), "replay %d: %s" % (i, k)
        say("graph B=%d S=%d replay %d: bit-identical to the eager step" % (B, num_splits, i))
        lens += 1
        oracle.paged_kv_append(kn, vn, W.newest_row_slots(lens, c.block_tables, c.BS), kp_o, vp_o)
    # the last replay against the oracle on the state it advanced itself
    assert np.array_equal(g_state["cl"].cpu().numpy(), lens)
    ref = oracle.decode_attention(q, kp_o, vp_o, c.block_tables, lens, c.scale)
    assert_close(g_state["out"].cpu().numpy(), ref, "graph B=%d S=%d last replay" % (B, num_splits))
    assert np.array_equal(g_state["kp"].cpu().numpy().view(np.uint16), kp_o.view(np.uint16))
    assert np.array_equal(g_state["vp"].cpu().numpy().view(np.uint16), vp_o.view(np.uint16))


@pytest.mark.parametrize("B", [4, 40])
def test_decode_step_qkv_graph_replays_follow_device_state(torch_cuda, B):
    """pkv_paged_decode_step_qkv captured once and replayed with new QKV rows and growing lengths: one launch for 4
    sequences, the QKV kernel then attention for 40 (320 workgroups)."""
    from paged_kv_decode_04_amd import pkv
    from test_gpu_qkv import assert_fp16_of
    torch = torch_cuda
    rng = np.random.default_rng(830 + B)
    lens0 = rng.integers(16, 120, B).astype(np.int32)
    c = W.build_qkv_case("graph", B, 32, 8, 128, 16, np.ones(B, np.int32), lens0 + STEPS - 1, 831 + B)
    vc = c.varlen
    width = (vc.Hq + 2 * vc.Hkv) * vc.D

    def state():
        return dict(qkv=torch.zeros((B, width), dtype=torch.float16, device="cuda"), qw=_dev(torch, c.q_norm_w),
                    kw=_dev(torch, c.k_norm_w), cos=_dev(torch, c.cos), sin=_dev(torch, c.sin),
                    kp=_dev(torch, vc.k_pool), vp=_dev(torch, vc.v_pool), bt=_dev(torch, vc.block_tables),
                    cl=_dev(torch, lens0), q=torch.zeros((B, vc.Hq, vc.D), dtype=torch.float16, device="cuda"),
                    out=torch.empty((B, vc.Hq, vc.D), dtype=torch.float16, device="cuda"))

    def step(st):
        pkv.paged_decode_step_qkv(st["qkv"], st["qw"], st["kw"], st["cos"], st["sin"], st["kp"], st["vp"], st["bt"],
                                  st["cl"], vc.Hq, vc.scale, c.eps, c.qk_mode, q_out=st["q"], out=st["out"],
                                  num_splits=1)

    g_state, e_state = state(), state()
    stream = torch.cuda.Stream()
    warm = state()
    with torch.cuda.stream(stream):
        step(warm)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(g_state)
    torch.cuda.synchronize()
    for k in ("kp", "vp", "out", "q"):
        g_state[k].copy_(e_state[k])
    kp_o, vp_o = vc.k_pool.copy(), vc.v_pool.copy()
    lens = lens0.copy()
    for i in range(STEPS):
        qkv = (2.0 * rng.standard_normal((B, width))).astype(np.float16)
        for st in (g_state, e_state):
            st["cl"].add_(1)
            st["qkv"].copy_(torch.from_numpy(qkv))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e_state)
        torch.cuda.synchronize()
        for k in ("out", "q", "kp", "vp"):
            assert torch.equal(g_state[k].view(torch.int16), e_state[k].view(torch.int16)), "replay %d: %s" % (i, k)
        say("graph step_qkv B=%d replay %d: bit-identical to the eager step" % (B, i))
        # the oracle's own step on its own state
        lens += 1
        q64, k64, slots = oracle.qkv_norm_rope_paged(qkv, c.q_norm_w, c.k_norm_w, c.cos, c.sin,
                                                     np.arange(B + 1, dtype=np.int32), lens - 1, lens - 1,
                                                     vc.block_tables, kp_o, vp_o, c.eps, c.qk_mode)
        k16 = k64.astype(np.float16)
        for t, slot in enumerate(slots):
            W.set_k_row(kp_o, int(slot) // vc.BS, slice(None), int(slot) % vc.BS, k16[t])
    ref = oracle.decode_attention(q64.astype(np.float16), kp_o, vp_o, vc.block_tables, lens, vc.scale)
    assert_close(g_state["out"].cpu().numpy(), ref, "graph step_qkv B=%d last replay" % B)
    assert_fp16_of(g_state["q"].cpu().numpy(), q64, "graph step_qkv B=%d last q_out" % B)


def test_varlen_step_graph_replays_follow_device_state(torch_cuda):
    """pkv_paged_varlen_step (one launch: 4 sequences x 8 kv heads) captured once and replayed while every sequence
    verifies 3 new rows per step: positions advance by 3, new q and K/V rows arrive."""
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    B, Hq, Hkv, D, BS, QL = 4, 32, 8, 128, 16, 3
    pos0 = np.array([40, 15, 77, 0], dtype=np.int32)
    c = W.build_varlen_case("graph", B, Hq, Hkv, D, BS, np.full(B, QL, np.int32), pos0 + QL * (STEPS - 1), 841,
                            poison_new=False)  # tables hold the grown sequences
    rng = np.random.default_rng(842)
    cu = np.arange(0, B * QL + 1, QL, dtype=np.int32)

    def state():
        return dict(q=torch.zeros((B * QL, Hq, D), dtype=torch.float16, device="cuda"),
                    kn=torch.zeros((B * QL, Hkv, D), dtype=torch.float16, device="cuda"),
                    vn=torch.zeros((B * QL, Hkv, D), dtype=torch.float16, device="cuda"),
                    kp=_dev(torch, c.k_pool), vp=_dev(torch, c.v_pool), bt=_dev(torch, c.block_tables),
                    cu=_dev(torch, cu), pos=_dev(torch, pos0 - QL),
                    out=torch.empty((B * QL, Hq, D), dtype=torch.float16, device="cuda"))

    def step(st):
        pkv.paged_varlen_step(st["q"], st["kn"], st["vn"], st["kp"], st["vp"], st["bt"], st["cu"], st["pos"], c.scale,
                              QL, out=st["out"], num_splits=1)

    g_state, e_state = state(), state()
    stream = torch.cuda.Stream()
    warm = state()
    warm["pos"].add_(QL)
    with torch.cuda.stream(stream):
        step(warm)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step(g_state)
    torch.cuda.synchronize()
    for k in ("kp", "vp", "out"):
        g_state[k].copy_(e_state[k])
    kp_o, vp_o = c.k_pool.copy(), c.v_pool.copy()
    pos = pos0 - QL
    for i in range(STEPS):
        q = rng.standard_normal((B * QL, Hq, D)).astype(np.float16)
        kn = rng.standard_normal((B * QL, Hkv, D)).astype(np.float16)
        vn = rng.standard_normal((B * QL, Hkv, D)).astype(np.float16)
        for st in (g_state, e_state):
            st["pos"].add_(QL)
            st["q"].copy_(torch.from_numpy(q))
            st["kn"].copy_(torch.from_numpy(kn))
            st["vn"].copy_(torch.from_numpy(vn))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(e_state)
        torch.cuda.synchronize()
        for k in ("out", "kp", "vp"):
            assert torch.equal(g_state[k].view(torch.int16), e_state[k].view(torch.int16)), "replay %d: %s" % (i, k)
        say("graph varlen step replay %d: bit-identical to the eager step" % i)
        pos = pos + QL
        slots = np.array([int(c.block_tables[s, (int(pos[s]) + j) // BS]) * BS + (int(pos[s]) + j) % BS
                          for s in range(B) for j in range(QL)], dtype=np.int32)
        oracle.paged_kv_append(kn, vn, slots, kp_o, vp_o)
    assert np.array_equal(g_state["pos"].cpu().numpy(), pos)
    ref = oracle.varlen_attention(q, kp_o, vp_o, c.block_tables, cu, pos, c.scale)
    assert_close(g_state["out"].cpu().numpy(), ref, "graph varlen step last replay")
    assert np.array_equal(g_state["kp"].cpu().numpy().view(np.uint16), kp_o.view(np.uint16))
    assert np.array_equal(g_state["vp"].cpu().numpy().view(np.uint16), vp_o.view(np.uint16))


def test_single_pass_capture_of_a_multi_round_grid_needs_no_warm_up(torch_cuda):
    """A single pass over 40 x 8 workgroups captured on a stream no call has used: the longest-first order would
    need the library workspace to grow, which capture forbids, so the captured call runs in id order instead of
    failing; its replay matches the eager result bit for bit."""
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    c = W.small_case(851, 40, 16, 8, 128, 16, tuple(1 + (53 * i) % 500 for i in range(40)))
    st = _state(torch, c, c.context_lens)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pkv.paged_decode_attention(st["q"], st["kp"], st["vp"], st["bt"], st["cl"], c.scale, out=st["out"],
                                   num_splits=1)
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
        torch.cuda.synchronize()
    eager = pkv.paged_decode_attention(st["q"], st["kp"], st["vp"], st["bt"], st["cl"], c.scale, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(st["out"].view(torch.int16), eager.view(torch.int16))


def test_capture_needing_a_new_workspace_fails_cleanly(torch_cuda):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    c = W.small_case(821, 2, 8, 2, 64, 16, (300, 40))
    st = _state(torch, c, c.context_lens)
    stream = torch.cuda.Stream()  # no call has sized this stream's workspace
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(pkv.PkvError) as e:
        with torch.cuda.graph(graph, stream=stream):
            pkv.paged_decode_attention(st["q"], st["kp"], st["vp"], st["bt"], st["cl"], c.scale, out=st["out"],
                                       num_splits=4)
    assert e.value.code == pkv.PKV_EWORKSPACE
    torch.cuda.synchronize()


def test_replay_after_the_workspace_grew_uses_a_live_buffer(torch_cuda):
    """A split-K call captured against the stream's library workspace, then a larger eager call on the same stream
    that makes the workspace grow: the captured graph still names the old buffer, which the library keeps alive, so
    replays (with fresh allocations made after the growth in between) stay correct against the oracle and leave
    those allocations untouched."""
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    small = W.small_case(861, 4, 32, 8, 128, 16, (700, 90, 333, 1024))
    big = W.small_case(862, 48, 32, 8, 128, 16, tuple(200 + (97 * i) % 1800 for i in range(48)))
    st = _state(torch, small, small.context_lens)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):  # sizes this stream's workspace for the small shape
        pkv.paged_decode_attention(st["q"], st["kp"], st["vp"], st["bt"], st["cl"], small.scale, out=st["out"],
                                   num_splits=3)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        pkv.paged_decode_attention(st["q"], st["kp"], st["vp"], st["bt"], st["cl"], small.scale, out=st["out"],
                                   num_splits=3)
    torch.cuda.synchronize()
    bst = _state(torch, big, big.context_lens)
    with torch.cuda.stream(stream):  # needs far more split partials: the workspace grows
        big_out = pkv.paged_decode_attention(bst["q"], bst["kp"], bst["vp"], bst["bt"], bst["cl"], big.scale,
                                             num_splits=8)
    stream.synchronize()
    canary = torch.full((1 << 20,), 0x5A5A, dtype=torch.int32, device="cuda")  # allocated after the growth
    ref_small = oracle.decode_attention(small.q, small.k_pool, small.v_pool, small.block_tables, small.context_lens,
                                        small.scale)
    for i in range(3):
        st["out"].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_close(st["out"].cpu().numpy(), ref_small, "replay %d after the workspace grew" % i)
    assert bool((canary == 0x5A5A).all())
    ref_big = oracle.decode_attention(big.q, big.k_pool, big.v_pool, big.block_tables, big.context_lens, big.scale)
    assert_close(big_out.cpu().numpy(), ref_big, "the call that grew the workspace")
