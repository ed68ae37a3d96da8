"""The worst case of fp16 softmax weights in the P.V product, built on purpose.

The matrix-core P.V product takes the weights p = 2^(s' - m) rounded once to fp16, while the running sum l keeps the
f32 p.  A normal fp16 rounding moves p by up to 2^-11 of itself (the most just above a power of two), so the output
moves by at most 2^-11 * sum_j p_j |v_j| / sum_j p_j <= 2^-11 * max|v|; the errors cancel unless every weight sits
just off a rounding midpoint and V's sign follows the direction each weight rounds.  The cases below do that, at
|v| = 4: the bound is 1.953e-3, under the 2e-3 attention bar (which the case would break only for |v| > 4.1), and the
kernels must land on the single-rounding model of the case (plus the fp16 output rounding) -- a kernel whose
weights were rounded differently, or whose l disagreed with them, would not.

These cases put the weights there: with scale = ln 2 (in f32) the kernels' log2-domain scale is exactly 1,
q = e0 + e1 and a key (-1, b) has the score s' = b - 1 exactly (fp16 b, exact f32 sum), so p = 2^(b - 1) lands 1e-6
below or above the midpoint 0.5 + 2^-12 between the fp16 values 0.5 and 0.5 + 2^-11; the keys below round down and
carry v = -4, those above round up and carry v = +4.  One key with score 0 (and v = 0) in the first unit each wave
reads keeps every wave's running max at 0, so every weight is rounded where it was placed.  The reference output is
small (1.6e-2 and 0.24), so the bars are absolute.
"""
import math

import numpy as np
import pytest

import oracle
from paged_kv_decode_04_amd import workloads as W

BAR = 2e-3
MID = 0.5 + 2.0 ** -12  # the rounding midpoint between the fp16 values 0.5 and 0.5 + 2^-11
SCALE = float(np.float32(math.log(2.0)))


def _offset(p_target):
    """The fp16 b whose score b - 1 gives p = 2^(b - 1) nearest p_target."""
    return np.float16(math.log2(p_target) + 1.0)


B_DOWN, B_UP = _offset(MID - 2.0 ** -20), _offset(MID + 2.0 ** -20)


def aligned_case(L, max_rows):
    """One sequence, one kv head and one query head, D = 128, BS = 16: rows in max_rows have score 0 and v = 0, the
    others alternate between rounding down with v = -4 and up with v = +4."""
    D, BS = 128, 16
    nb = (L + BS - 1) // BS
    c = W.build_case("fp16_p_worst", 1, 1, 1, D, BS, [L], nb + 4, nb, SCALE, seed=4242, with_append=False)
    q = np.zeros((1, 1, D), np.float16)
    q[0, 0, :2] = 1.0
    c.q = q
    zero = np.zeros(D, np.float16)
    down_k, up_k = zero.copy(), zero.copy()
    down_k[:2] = (-1.0, B_DOWN)
    up_k[:2] = (-1.0, B_UP)
    for j in range(L):
        blk, off = int(c.block_tables[0, j // BS]), j % BS
        if j in max_rows:
            k, v = zero, zero
        elif j % 2:
            k, v = down_k, np.full(D, -4.0, np.float16)
        else:
            k, v = up_k, np.full(D, 4.0, np.float16)
        W.set_k_row(c.k_pool, blk, 0, off, k)
        W.set_v_row(c.v_pool, blk, 0, off, v)
    return c


def modelled_error(L, max_rows):
    """The output error of f32 weights rounded to fp16 with l summed from the unrounded weights (f64 model)."""
    p = {True: 2.0 ** (float(B_DOWN) - 1.0), False: 2.0 ** (float(B_UP) - 1.0)}
    num_exact = num_rounded = l = 0.0
    for j in range(L):
        if j in max_rows:
            l += 1.0
            continue
        down = bool(j % 2)
        v = -4.0 if down else 4.0
        num_exact += p[down] * v
        num_rounded += float(np.float16(p[down])) * v
        l += p[down]
    return (num_rounded - num_exact) / l


def test_the_case_rounds_every_weight_the_way_its_value_points():
    """CPU check of the construction: the two scores are exact in f32, their weights lie on either side of the
    midpoint by more than the f32 exponential's error, fp16 rounds them apart, and the modelled error is within the
    bound and close to it."""
    f32 = np.float32
    assert f32(f32(SCALE) * f32(1.44269504088896340736)) == f32(1.0)
    for b, down in ((B_DOWN, True), (B_UP, False)):
        s = f32(f32(-1.0) + f32(b))
        assert float(s) == float(b) - 1.0  # exact sum
        p = 2.0 ** float(s)
        assert abs(p - MID) > 5e-7  # far beyond a few f32 ulps (6e-8 near 0.5)
        r = float(np.float16(p))
        assert (r < p) == down and abs(r - p) > 2.0 ** -12 - 2.0 ** -19
    rows = set(range(0, 128, 16))
    err = modelled_error(2048, rows)
    assert 0.95 * 2.0 ** -11 * 4 < abs(err) <= 2.0 ** -11 * 4


@pytest.mark.gpu
@pytest.mark.parametrize("what, L, max_rows, splits", [
    ("first unit of every wave", 2048, set(range(0, 128, 16)), (1,)),
    ("every unit", 2048, set(range(0, 2048, 16)), (1, 0, 4)),
])
def test_fp16_weights_aligned_worst_case(what, L, max_rows, splits):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_decode_04_amd import pkv
    pkv.load()
    c = aligned_case(L, max_rows)
    ref = oracle.decode_attention(c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens, c.scale)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    d = [dev(x) for x in (c.q, c.k_pool, c.v_pool, c.block_tables, c.context_lens)]
    model = modelled_error(L, max_rows)
    for S in splits:
        out = pkv.paged_decode_attention(*d, c.scale, num_splits=S).cpu().numpy().astype(np.float64)
        err = float(np.abs(out - ref).max())
        print("[precision] %s, num_splits=%d: max|err| %.3e (f16-weight model %.3e, bound %.3e), max|ref| %.1e"
              % (what, S, err, abs(model), 2.0 ** -11 * 4, float(np.abs(ref).max())), flush=True)
        assert np.all(np.isfinite(out))
        assert err <= BAR and err <= 2.0 ** -11 * 4
        assert abs(err - abs(model)) <= 1e-4  # the single-rounding model, up to the fp16 output rounding
