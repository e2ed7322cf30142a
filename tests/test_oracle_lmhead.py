"""Pins of the oracle's logit projection (sv_oracle_lmhead_logits) and of its
greedy verify on double-precision logits.

The projection logits[i][v] = sum_k hidden[i][k] * weight[v][k] is pinned
against things other than itself: numpy's float64 matrix product on inputs
where every sum is exact (a library routine; any summation order gives the same
value there), one-hot rows that select a single weight column or hidden entry
(a transposed operand or a wrong stride fails these at non-square shapes), and
exact scaling by powers of two.  The greedy rule on float64 logits is pinned to
numpy's first-occurrence argmax and to the established float32 path."""
import numpy as np
import pytest

from oracle import get as get_oracle


def _bits(a):
    """bf16 bit patterns of float32 values that bf16 holds exactly."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    assert np.array_equal(a.view(np.uint32) & 0xFFFF, np.zeros(a.shape, np.uint32)), "not bf16-exact"
    return (a.view(np.uint32) >> 16).astype(np.uint16)


@pytest.fixture(scope="module")
def o():
    return get_oracle()


def _int_case(seed, M, H, V, R=44):
    rng = np.random.default_rng(seed)
    h = rng.integers(-R, R + 1, (M, H)).astype(np.float32) / 16.0
    w = rng.integers(-R, R + 1, (V, H)).astype(np.float32) / 1024.0
    return h, w


@pytest.mark.parametrize("M,H,V", [(7, 48, 33), (1, 1, 1), (5, 200, 3), (12, 64, 129)])
def test_projection_equals_numpy_on_exact_inputs(o, M, H, V):
    h, w = _int_case(M * 1000 + H + V, M, H, V)
    got = o.lmhead_logits(_bits(h), _bits(w), threads=3)
    ref = h.astype(np.float64) @ w.astype(np.float64).T
    assert got.shape == (M, V)
    assert np.array_equal(got, ref)


def test_projection_row_subset_and_threads(o):
    h, w = _int_case(5, 9, 32, 17)
    rows = np.array([8, 0, 3, 3], np.int32)
    full = o.lmhead_logits(_bits(h), _bits(w))
    sub = o.lmhead_logits(_bits(h), _bits(w), rows=rows, threads=5)
    assert np.array_equal(sub, full[rows])


def test_one_hot_hidden_rows_select_weight_columns(o):
    """hidden row i = e_{k_i}: logits[i] is column k_i of the weight (weight[:, k_i])."""
    rng = np.random.default_rng(1)
    M, H, V = 6, 10, 23
    w = (rng.integers(-100, 101, (V, H)) / 64.0).astype(np.float32)
    ks = rng.integers(0, H, M)
    h = np.zeros((M, H), np.float32)
    h[np.arange(M), ks] = 1.0
    got = o.lmhead_logits(_bits(h), _bits(w))
    for i in range(M):
        assert np.array_equal(got[i], w[:, ks[i]].astype(np.float64))


def test_one_hot_weight_rows_select_hidden_entries(o):
    """weight row v = c_v * e_{pi(v)}: logits[:, v] = c_v * hidden[:, pi(v)]."""
    rng = np.random.default_rng(2)
    M, H, V = 5, 7, 19
    h = (rng.integers(-100, 101, (M, H)) / 8.0).astype(np.float32)
    pi = rng.integers(0, H, V)
    c = rng.choice(np.array([0.5, -2.0, 4.0, 1.0], np.float32), V)
    w = np.zeros((V, H), np.float32)
    w[np.arange(V), pi] = c
    got = o.lmhead_logits(_bits(h), _bits(w))
    assert np.array_equal(got, h[:, pi].astype(np.float64) * c.astype(np.float64))


def test_projection_scales_by_powers_of_two(o):
    h, w = _int_case(3, 4, 40, 11)
    base = o.lmhead_logits(_bits(h), _bits(w))
    assert np.array_equal(o.lmhead_logits(_bits(h * 2.0), _bits(w)), 2.0 * base)
    assert np.array_equal(o.lmhead_logits(_bits(h), _bits(w * 0.25)), 0.25 * base)
    assert np.array_equal(o.lmhead_logits(_bits(-h), _bits(w)), -base)


def test_greedy_on_float64_logits_matches_numpy_and_float32(o):
    """The greedy rule applied to double logits: accepted prefix = the drafts
    that equal numpy's first-occurrence argmax; equals the float32 path when the
    logits are float32-exact.  Duplicated weight rows give exact ties that the
    lowest index must win."""
    B, n, H, V = 6, 3, 24, 50
    h, w = _int_case(4, B * (n + 1), H, V)
    w[31] = w[7]     # twin columns: equal logits in every row
    w[2] = w[40]
    for r in (0, 5, 13):         # rows whose top is the tied pair (7, 31)
        h[r] = w[7] * 64.0
    for r in (6, 8, 17):         # rows whose top is the tied pair (2, 40)
        h[r] = w[2] * 64.0
    z = o.lmhead_logits(_bits(h), _bits(w)).reshape(B, n + 1, V)
    am = z.argmax(-1)  # first occurrence
    assert (am.reshape(-1)[[0, 5, 13]] == 7).all() and (am.reshape(-1)[[6, 8, 17]] == 2).all()
    x = am[:, :n].copy().astype(np.int32)
    x[1, 1] = 31 if am[1, 1] == 7 else (x[1, 1] + 1) % V   # the twin: rejected
    x[2, 0] = 40 if am[2, 0] == 2 else (x[2, 0] + 1) % V
    lens = np.array([3, 3, 3, 2, 0, 1], np.int32)
    r64 = o.verify_greedy(z, x, lens)
    r32 = o.verify_greedy(z.astype(np.float32), x, lens)
    assert np.array_equal(r64["accepted_len"], r32["accepted_len"])
    assert np.array_equal(r64["emitted"], r32["emitted"])
    for b in range(B):
        k = 0
        while k < lens[b] and x[b, k] == am[b, k]:
            k += 1
        assert r64["accepted_len"][b] == k
        assert r64["emitted"][b, k] == am[b, k]
    assert r64["accepted_len"][1] == 1 and r64["emitted"][1, 1] == 7
    assert r64["accepted_len"][2] == 0 and r64["emitted"][2, 0] == 2


def _pins_hold(orc):
    """The projection pins above, as one boolean (for the negative controls)."""
    ok = True
    for M, H, V in [(7, 48, 33), (12, 64, 129)]:
        h, w = _int_case(M * 1000 + H + V, M, H, V)
        ok &= np.array_equal(orc.lmhead_logits(_bits(h), _bits(w)), h.astype(np.float64) @ w.astype(np.float64).T)
    rng = np.random.default_rng(1)
    M, H, V = 6, 10, 23
    w = (rng.integers(-100, 101, (V, H)) / 64.0).astype(np.float32)
    ks = rng.integers(0, H, M)
    h = np.zeros((M, H), np.float32)
    h[np.arange(M), ks] = 1.0
    got = orc.lmhead_logits(_bits(h), _bits(w))
    ok &= all(np.array_equal(got[i], w[:, ks[i]].astype(np.float64)) for i in range(M))
    return bool(ok)


def test_projection_pins_hold_for_the_oracle(o):
    assert _pins_hold(o)


@pytest.mark.parametrize("plant", [4, 5])
def test_planted_projection_mistakes_fail_the_pins(planted, plant):
    """Oracle builds with a dropped product (4) or a transposed weight index (5)
    must fail the pins."""
    assert not _pins_hold(planted(plant))

