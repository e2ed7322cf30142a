"""Pins of the oracle's greedy tree verification (EAGLE section of
"Accelerating Sonar through speculation": the longest suitable candidate sequence
is kept and one more target token is appended; greedy reading: a node is suitable
when its token is the target's argmax at its parent and its parent is suitable).

- a chain tree (every node below the previous one) is the linear greedy rule,
  itself pinned by a numpy-argmax prefix match;
- a brute force over every root-to-node path, each checked node by node with
  numpy.argmax (first occurrence), agrees on random trees with many ties;
- a star tree accepts at most one node;
- bad parents and out-of-range tokens are flagged, never read out of bounds;
- oracle builds with a planted mistake fail these pins.
"""
import numpy as np
import pytest

import oracle as orc


@pytest.fixture(scope="module")
def o():
    return orc.Oracle()


def _random_case(rng, B, n, V, ties=True):
    z = (rng.integers(-3, 4, (B, n + 1, V)) if ties else rng.standard_normal((B, n + 1, V))).astype(np.float32)
    par = np.zeros((B, n), np.int32)
    x = np.zeros((B, n), np.int32)
    for b in range(B):
        for j in range(n):
            par[b, j] = rng.integers(0, j + 1)
            g = int(np.argmax(z[b, par[b, j]]))
            x[b, j] = g if rng.random() < 0.75 else rng.integers(0, V)
    L = rng.integers(0, n + 1, B).astype(np.int32)
    return z, x, par, L


def _brute(z, x, par, L):
    """Every root-to-node path (node j + 1 holds x[j] below node par[j]), checked
    node by node against numpy's first-occurrence argmax of the parent's row; the
    longest accepted path, the lowest end node among equally long ones."""
    B, n1, V = z.shape
    n = n1 - 1
    acc = np.zeros(B, np.int32)
    emi = np.full((B, n + 1), -1, np.int32)
    path = np.full((B, n), -1, np.int32)
    for b in range(B):
        best = ([], 0)
        for end in range(1, int(L[b]) + 1):
            chain, node, ok = [], end, True
            while node != 0:
                p = int(par[b, node - 1])
                if not (0 <= p < node):
                    ok = False
                    break
                chain.append(node)
                node = p
            if not ok:
                continue
            chain.reverse()
            if all(x[b, c - 1] == int(np.argmax(z[b, int(par[b, c - 1])])) for c in chain):
                if len(chain) > len(best[0]):
                    best = (chain, end)
        chain = best[0]
        acc[b] = len(chain)
        for d, c in enumerate(chain):
            path[b, d] = c
            emi[b, d] = x[b, c - 1]
        emi[b, len(chain)] = int(np.argmax(z[b, chain[-1] if chain else 0]))
    return acc, emi, path


def _pins_hold(oo):
    ok = True
    rng = np.random.default_rng(31)
    for B, n, V, ties in [(40, 8, 6, True), (30, 12, 50, True), (20, 6, 200, False), (10, 0, 9, True)]:
        z, x, par, L = _random_case(rng, B, n, V, ties)
        r = oo.verify_tree_greedy(z, x, par, L)
        a, e, pth = _brute(z, x, par, L)
        ok &= np.array_equal(r["accepted_len"], a) and np.array_equal(r["emitted"], e)
        ok &= np.array_equal(r["path"], pth)
    # a chain is the linear greedy rule
    z, x, _, L = _random_case(rng, 50, 7, 8, True)
    chain = np.tile(np.arange(7, dtype=np.int32), (50, 1))
    r = oo.verify_tree_greedy(z, x, chain, L)
    g = oo.verify_greedy(z, x, L)
    ok &= np.array_equal(r["accepted_len"], g["accepted_len"]) and np.array_equal(r["emitted"], g["emitted"])
    return bool(ok)


def test_pins_hold(o):
    assert _pins_hold(o)


def test_chain_tree_is_the_linear_greedy_rule(o):
    rng = np.random.default_rng(5)
    for B, n, V in [(64, 4, 7), (33, 9, 100), (8, 0, 5)]:
        z, x, _, L = _random_case(rng, B, n, V, True)
        chain = np.tile(np.arange(n, dtype=np.int32), (B, 1))
        r = o.verify_tree_greedy(z, x, chain, L)
        g = o.verify_greedy(z, x, L)
        assert np.array_equal(r["accepted_len"], g["accepted_len"])
        assert np.array_equal(r["emitted"], g["emitted"])
        for b in range(B):  # the path of a chain is nodes 1..k
            k = int(r["accepted_len"][b])
            assert r["path"][b, :k].tolist() == list(range(1, k + 1)) and (r["path"][b, k:] == -1).all()


def test_brute_force_on_random_trees(o):
    rng = np.random.default_rng(6)
    for B, n, V, ties in [(60, 10, 5, True), (40, 15, 30, True), (20, 8, 1000, False)]:
        z, x, par, L = _random_case(rng, B, n, V, ties)
        r = o.verify_tree_greedy(z, x, par, L)
        a, e, pth = _brute(z, x, par, L)
        assert np.array_equal(r["accepted_len"], a)
        assert np.array_equal(r["emitted"], e)
        assert np.array_equal(r["path"], pth)
        assert (r["seq_flags"] == 0).all()


def test_star_tree_accepts_at_most_one_node(o):
    rng = np.random.default_rng(7)
    B, n, V = 50, 6, 4
    z = rng.integers(-2, 3, (B, n + 1, V)).astype(np.float32)
    x = rng.integers(0, V, (B, n)).astype(np.int32)
    par = np.zeros((B, n), np.int32)
    L = np.full(B, n, np.int32)
    r = o.verify_tree_greedy(z, x, par, L)
    for b in range(B):
        g = int(np.argmax(z[b, 0]))
        hits = [j + 1 for j in range(n) if x[b, j] == g]
        assert r["accepted_len"][b] == (1 if hits else 0)
        if hits:
            assert r["path"][b, 0] == hits[0]  # the lowest node among equally deep ones
            assert r["emitted"][b, 0] == g and r["emitted"][b, 1] == int(np.argmax(z[b, hits[0]]))
        else:
            assert r["emitted"][b, 0] == g


def test_bad_parents_and_tokens_are_flagged(o):
    z = np.zeros((3, 4, 5), np.float32)
    z[:, :, 2] = 1.0  # argmax 2 everywhere
    x = np.array([[2, 2, 2], [2, 9, 2], [2, 2, 2]], np.int32)
    par = np.array([[0, 1, 2], [0, 1, 1], [0, 5, -1]], np.int32)
    L = np.array([3, 3, 3], np.int32)
    r = o.verify_tree_greedy(z, x, par, L)
    assert r["accepted_len"].tolist() == [3, 2, 1]
    assert r["path"][1].tolist() == [1, 3, -1]  # node 2 holds token 9: out of range, never accepted
    assert r["seq_flags"].tolist() == [0, orc.FLAG_TOKEN_OOR, orc.FLAG_BAD_PARENT]
    r = o.verify_tree_greedy(z, x, par, np.array([-1, 4, 1], np.int32))
    assert r["accepted_len"].tolist() == [0, 2, 1]
    assert r["seq_flags"].tolist() == [orc.FLAG_LEN_CLAMPED, orc.FLAG_LEN_CLAMPED | orc.FLAG_TOKEN_OOR, 0]


@pytest.mark.parametrize("plant", [6, 7])
def test_planted_tree_mistakes_fail_the_pins(planted, plant):
    """Oracle builds that compare a node's token with its own row's argmax (6) or
    ignore whether its parent was accepted (7) must fail the pins."""
    assert not _pins_hold(planted(plant))
