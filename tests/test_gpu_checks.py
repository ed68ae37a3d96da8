"""The cold-path input checks (pkv_check_decode_inputs, pkv_check_varlen_inputs, pkv_check_slot_mapping) on the GPU:
valid inputs report nothing; planted problems are counted exactly as the entry points' rules define them (the
expected counts are written out here from those rules), and entries a call would not read are not counted."""
import numpy as np
import pytest

from paged_kv_decode_04_amd import workloads as W
from test_gpu_parity import say, torch_cuda, _dev  # noqa: F401  (fixture and helpers)

pytestmark = pytest.mark.gpu

NONE = np.iinfo(np.int32).max


def _expected_decode(bt, lens, N, BS, window=0):
    B, M = bt.shape
    bad_len = bad_ent = 0
    first = NONE
    for s in range(B):
        L = int(lens[s])
        bad = L < 0 or L > M * BS
        n_ent = 0
        if not bad:
            lo = L - window if 0 < window < L else 0
            for j in range(lo // BS, (L + BS - 1) // BS):
                n_ent += not (0 <= bt[s, j] < N)
        bad_len += bad
        bad_ent += n_ent
        if (bad or n_ent) and first == NONE:
            first = s
    return [bad_len, bad_ent, first, 0]


def _report(torch, fn):
    r = fn()
    torch.cuda.synchronize()
    return r.cpu().numpy().tolist()


def test_decode_checks(torch_cuda):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    c = W.small_case(1501, 5, 8, 2, 64, 16, (40, 17, 100, 1, 64))
    kp, vp = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    run = lambda bt, lens, window=0: _report(torch, lambda: pkv.check_decode_inputs(
        kp, vp, _dev(torch, bt), _dev(torch, lens), window=window))
    assert run(c.block_tables, c.context_lens) == [0, 0, NONE, 0]
    bt, lens = c.block_tables.copy(), c.context_lens.copy()
    lens[3] = -1                      # a negative length
    lens[4] = c.M * c.BS + 1          # past the table's capacity
    bt[2, 5] = -1                     # a read entry (sequence 2 reads blocks 0..6)
    bt[2, 6] = c.N                    # another
    bt[0, c.M - 1] = 10 ** 6          # past sequence 0's last block: never read
    got = run(bt, lens)
    assert got == _expected_decode(bt, lens, c.N, c.BS) == [2, 2, 2, 0], got
    # with a window of 20 rows sequence 2 reads only blocks 5 and 6 (rows 80..99); a bad early entry is not read
    bt2 = c.block_tables.copy()
    bt2[2, 0] = -1
    assert run(bt2, c.context_lens, window=20) == [0, 0, NONE, 0]
    assert run(bt2, c.context_lens) == _expected_decode(bt2, c.context_lens, c.N, c.BS) == [0, 1, 2, 0]
    say("decode input checks: ok")


def test_varlen_checks(torch_cuda):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    vc = W.build_varlen_case("chk", 3, 8, 2, 64, 16, (3, 0, 5), (10, 40, 30), 1502)
    kp, vp = _dev(torch, vc.k_pool), _dev(torch, vc.v_pool)
    run = lambda bt, cu, pos, T: _report(torch, lambda: pkv.check_varlen_inputs(
        kp, vp, _dev(torch, bt), _dev(torch, np.asarray(cu, np.int32)), _dev(torch, np.asarray(pos, np.int32)), T))
    cu, pos, T = vc.cu_seqlens_q, vc.pos_offsets, vc.T
    assert run(vc.block_tables, cu, pos, T) == [0, 0, NONE, 0]
    assert run(vc.block_tables, [1, 3, 3, 8], pos, T) == [1, 0, 0, 0]          # cu[0] != 0
    assert run(vc.block_tables, [0, 3, 2, 8], pos, T) == [1, 0, 1, 0]          # decreasing
    assert run(vc.block_tables, cu, pos, T + 1) == [1, 0, 2, 0]                # cu[B] != T
    assert run(vc.block_tables, cu, [10, -1, 30], T) == [1, 0, 1, 0]           # negative position
    cap = vc.M * vc.BS
    assert run(vc.block_tables, cu, [10, 40, cap - 4], T) == [1, 0, 2, 0]      # runs past the capacity
    bt = vc.block_tables.copy()
    bt[2, 2] = -1                     # sequence 2 reads blocks 0..2 (rows 0..34)
    assert run(bt, cu, pos, T) == [0, 1, 2, 0]
    say("varlen input checks: ok")


def test_slot_checks(torch_cuda):
    from paged_kv_decode_04_amd import pkv
    torch = torch_cuda
    c = W.small_case(1503, 3, 8, 2, 64, 16, (40, 17, 100))
    kp, vp = _dev(torch, c.k_pool), _dev(torch, c.v_pool)
    run = lambda slots: _report(torch, lambda: pkv.check_slot_mapping(kp, vp, _dev(torch, np.asarray(slots,
                                                                                                     np.int32))))
    cap = c.N * c.BS
    assert run(c.slot_mapping) == [0, 0, NONE, 0]
    assert run([5, -1, cap, 7, cap + 100, -30]) == [0, 0, 2, 2]  # padding allowed, two slots out of the pool
    slots = np.arange(700, dtype=np.int32) % cap
    slots[[300, 650]] = cap
    assert run(slots) == [0, 0, 300, 2]                           # several workgroups
    say("slot checks: ok")


@pytest.mark.gpu
def test_stream_read_probe_reads_every_run_and_writes_its_outputs():
    """The floor probe (libpkvprobe.so): output chunk j of a workgroup carries the XOR of the words of the chunks its
    thread j read (chunks j, j + 512, ... of the run) and the index j, so a wrong offset or a dropped load shows."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ctypes, os
    lib = ctypes.CDLL(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                   "paged_kv_decode_04_amd", "libpkvprobe.so"))
    f = lib.pkv_probe_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 3 + [ctypes.c_int32, ctypes.c_int32,
                                                                             ctypes.c_void_p]
    rng = np.random.default_rng(5)
    len16 = np.array([0, 1, 7, 4096, 5000, 33], np.int64)
    off16 = np.concatenate([[0], np.cumsum(len16)[:-1]]).astype(np.int64)
    words = rng.integers(0, 2**32, size=int(len16.sum()) * 4, dtype=np.uint64).astype(np.uint32)
    x = torch.from_numpy(words.view(np.int32)).cuda()
    y = torch.zeros(len(len16) * 64 // 4, dtype=torch.int32, device="cuda")  # 64 bytes per workgroup
    # every device buffer stays referenced until the launch is done (a temporary's block could be handed to the
    # next allocation before the kernel reads it)
    off_d = torch.from_numpy(off16).cuda()
    len_d = torch.from_numpy(len16.astype(np.int32)).cuda()
    assert off_d.data_ptr() != len_d.data_ptr()
    rc = f(x.data_ptr(), x.numel() * 4, off_d.data_ptr(), len_d.data_ptr(), y.data_ptr(), len(len16), 64,
           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    got = y.cpu().numpy().view(np.uint32).reshape(len(len16), 4, 4)
    for g in range(len(len16)):
        run = words[off16[g] * 4:(off16[g] + len16[g]) * 4].reshape(-1, 4)
        for j in range(4):
            mine = run[j::512]
            acc = np.bitwise_xor.reduce(mine.reshape(-1)) if mine.size else np.uint32(0)
            assert got[g, j, 0] == acc and got[g, j, 1] == acc ^ 1 and got[g, j, 2] == acc ^ 2 and got[g, j, 3] == j
