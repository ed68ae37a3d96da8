"""Graph-replayable decode: a decode step captured once in a HIP graph (torch.cuda.graph) replays correctly while
the device-resident state moves on -- the context lengths grow by one each step, new q and new K/V rows arrive --
with the program's own eager work and synchronisations between replays.  Every replay is checked bit for bit
against the same step run eagerly on a separate copy of the state, and the last one against the oracle.
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


@pytest.mark.parametrize("num_splits", [1, 3])
def test_decode_step_graph_replays_follow_device_state(torch_cuda, num_splits):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    lens0 = np.array([100, 31, 47, 16], dtype=np.int32)
    c = W.small_case(811 + num_splits, 4, 32, 8, 128, 16, lens0 + STEPS)  # tables hold the grown sequences
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
        say("graph S=%d replay %d: bit-identical to the eager step" % (num_splits, i))
    # the last replay against the oracle, over the pools as the replays left them
    cl = g_state["cl"].cpu().numpy()
    ref = oracle.decode_attention(q, g_state["kp"].cpu().numpy(), g_state["vp"].cpu().numpy(), c.block_tables, cl,
                                  c.scale)
    assert_close(g_state["out"].cpu().numpy(), ref, "graph S=%d last replay" % num_splits)


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
