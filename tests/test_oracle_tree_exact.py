"""Pin of the oracle's sampling tree walk against brute force in exact-enough
arithmetic: SpecInfer's multi-step speculative sampling applied literally, with
every probability a Python ``Decimal`` carried to far more digits than the
smallest quantity the walk compares (target and draft rows of 6 tokens, so the
brute force is cheap).  At each node the children are tested in index order:
child j is kept iff u[j] < r(x_j) / q(x_j), r starting as the target's softmax
and, after each rejection, replaced by max(0, r - q) normalised; with no child
kept the token is drawn from r by inverse CDF with u[n]; a node without
children draws from the target's own row.

The rows are those where a walk's arithmetic is hardest: both rows on one top
token at low temperature, so that after two rejections at a node the weight of
the tokens the rows share is a second-order quantity (the product of two tails)
set against first-order ones, and p - lam q computed from its parts keeps none
of its digits.  Cases whose uniforms lie within 1e-9 of a decision boundary
(relative) are not compared, and are counted.  The linear rule is pinned the
same way, on the chain tree.
"""
from decimal import Decimal, localcontext

import numpy as np

GRID = 1.0 / 32.0   # relative logits on a grid exact in bf16 and binary32


def _softmax(row, T):
    m = max(Decimal(float(v)) for v in row if np.isfinite(v))
    e = [((Decimal(float(v)) - m) / T).exp() if np.isfinite(v) else Decimal(0) for v in row]
    S = sum(e)
    return [v / S for v in e]


def _draw(w, u):
    """Inverse CDF over weights w (summing to 1): index, relative margin."""
    t = Decimal(float(u))
    C = Decimal(0)
    for i, wi in enumerate(w):
        prev = C
        C += wi
        if C > t:
            return i, min(t - prev, C - t)
    return None, Decimal(0)


def exact_walk(zt, zd, x, par, L, T, u):
    """The walk of one sequence: (accepted length, emitted token after the
    kept path, the smallest margin of any decision, rejections at the drawing
    node)."""
    n = zd.shape[0]
    node, depth, margin = 0, 0, Decimal(1)
    Tq = Decimal(float(np.float32(T)))
    while True:
        kids = [j for j in range(L) if par[j] == node]
        r = _softmax(zt[node], Tq)
        if not kids:
            y, m = _draw(r, u[n])
            return depth, y, min(margin, m), 0
        q = _softmax(zd[node], Tq)
        kept, rejections = None, 0
        for j in kids:
            xj = int(x[j])
            ratio = r[xj] / q[xj] if q[xj] > 0 else Decimal("Infinity")
            uj = Decimal(float(u[j]))
            if ratio.is_finite():
                margin = min(margin, abs(uj - ratio) / max(ratio, Decimal(1e-300)))
            if uj < ratio:
                kept = j
                break
            rejections += 1
            res = [max(Decimal(0), a - b) for a, b in zip(r, q)]
            Z = sum(res)
            assert Z > 0
            r = [v / Z for v in res]
        if kept is None:
            y, m = _draw(r, u[n])
            return depth, y, min(margin, m), rejections
        node, depth = kept + 1, depth + 1


def _case(rng):
    """Rows of 6 tokens sharing the top token (one of them at random also shares
    a lower logit), a tree of 4 drafts with repeated and distinct siblings."""
    V, n = 6, 4
    zt = np.zeros((n + 1, V), np.float32)
    zd = np.zeros((n, V), np.float32)
    for k in range(n + 1):
        top = rng.integers(V)
        rel = -GRID * rng.integers(8, 96, V)
        rel[top] = 0.0
        zt[k] = rel + GRID * rng.integers(-64, 64)
        if k < n:
            d = -GRID * rng.integers(4, 96, V)
            d[top] = 0.0
            same = rng.random(V) < 0.3
            d[same] = rel[same]
            zd[k] = d + GRID * rng.integers(-64, 64)
    par = np.zeros(n, np.int32)
    for j in range(1, n):
        par[j] = rng.integers(0, j + 1) if rng.random() < 0.4 else par[j - 1]
    x = np.zeros(n, np.int32)
    for j in range(n):
        p = par[j]
        fav = int(np.argmax((zd[p] - zd[p].max()) - (zt[p] - zt[p].max())))
        x[j] = fav if rng.random() < 0.6 else rng.integers(V)
    return zt, zd, x, par


def test_tree_walk_matches_exact_brute_force(oracle):
    rng = np.random.default_rng(20261203)
    temps = [0.003, 0.01, 0.03, 0.1, 1.0]
    compared = deep = skipped = 0
    mism = []
    for case in range(300):
        zt, zd, x, par = _case(rng)
        T = temps[case % len(temps)]
        u = rng.random(5).astype(np.float32)
        rel = np.concatenate([(zt - zt.max(1, keepdims=True)).ravel(), (zd - zd.max(1, keepdims=True)).ravel()])
        digits = int(2.2 * float(-rel.min()) / T / 2.302) + 60
        with localcontext() as c:
            c.prec = digits
            c.Emin, c.Emax = -10 ** 9, 10 ** 9
            acc, y, margin, rej = exact_walk(zt, zd, x, par, 4, T, u)
        if margin < Decimal("1e-9"):
            skipped += 1
            continue
        o = oracle.verify_tree_sample(zt[None], zd[None], x[None], par[None], np.array([4], np.int32),
                                      np.array([T], np.float32), u[None])
        compared += 1
        deep += rej >= 2
        if int(o["accepted_len"][0]) != acc or int(o["emitted"][0, acc]) != y:
            mism.append((case, T, acc, y, int(o["accepted_len"][0]), int(o["emitted"][0, acc])))
    assert not mism, mism[:10]
    assert compared >= 270 and deep >= 30, (compared, deep, skipped)


def test_linear_rule_matches_exact_brute_force(oracle):
    """The linear rule (`verify_sample`: the first rejection ends the prefix and
    the token is drawn from max(0, p - q) normalised) on the same kind of rows,
    n = 3 drafts, against the brute force on the chain tree (node j + 1 below
    node j), which is the same rule."""
    rng = np.random.default_rng(777)
    temps = [0.003, 0.01, 0.03, 0.1, 1.0]
    compared = rejected = skipped = 0
    mism = []
    chain = np.array([0, 1, 2], np.int32)
    for case in range(300):
        zt, zd, _, _ = _case(rng)
        zt, zd = zt[:4], zd[:3]
        T = temps[case % len(temps)]
        x = np.array([int(np.argmax((zd[j] - zd[j].max()) - (zt[j] - zt[j].max()))) if rng.random() < 0.6
                      else int(rng.integers(6)) for j in range(3)], np.int32)
        L = int(rng.integers(0, 4))
        u = rng.random(4).astype(np.float32)
        rel = np.concatenate([(zt - zt.max(1, keepdims=True)).ravel(), (zd - zd.max(1, keepdims=True)).ravel()])
        with localcontext() as c:
            c.prec = int(2.2 * float(-rel.min()) / T / 2.302) + 60
            c.Emin, c.Emax = -10 ** 9, 10 ** 9
            acc, y, margin, rej = exact_walk(zt, zd, x, chain, L, T, u)
        if margin < Decimal("1e-9"):
            skipped += 1
            continue
        o = oracle.verify_sample(zt[None], zd[None], x[None], np.array([L], np.int32), np.array([T], np.float32),
                                 u[None])
        compared += 1
        rejected += acc < L
        if int(o["accepted_len"][0]) != acc or int(o["emitted"][0, acc]) != y:
            mism.append((case, T, L, acc, y, int(o["accepted_len"][0]), int(o["emitted"][0, acc])))
    assert not mism, mism[:10]
    assert compared >= 270 and rejected >= 60, (compared, rejected, skipped)
