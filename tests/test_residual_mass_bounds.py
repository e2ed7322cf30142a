"""The lower bounds of the residual mass that decide which form a draw's chunks
hand over, checked on random distributions (pure numpy; the bounds only pick a
form, the draw itself checks the mass it finds).

With S = sum exp((z - m) / T) a row's top token has probability 1 / S.  After a
rejection of x at lam = 1 the mass Z = sum max(0, p - q) = sum max(0, q - p) is at
least q(x) - p(x) and |1 / S_t - 1 / S_d|.  On a tree node after k rejections,
lam_{k+1} = lam_k + M_k, the next mass is at least M_k (q(x) - r_k(x)) for the
rejected x (r_k = max(0, p - lam_k q) / M_k), at least M_k / S_d - max(0, 1 / S_t -
lam_k / S_d), and at least 1 / S_t - lam_{k+1} / S_d."""
import numpy as np


def _rows(rng, V, T, close):
    zt = rng.normal(0.0, 3.0, V)
    zd = zt + rng.normal(0.0, close, V) if close else rng.normal(0.0, 3.0, V)
    if rng.random() < 0.5:  # a shared top token
        i = rng.integers(V)
        zt[i] = zt.max() + rng.uniform(0, 8)
        zd[i] = zd.max() + rng.uniform(0, 8)
    St = np.exp((zt - zt.max()) / T).sum()
    Sd = np.exp((zd - zd.max()) / T).sum()
    return np.exp((zt - zt.max()) / T) / St, np.exp((zd - zd.max()) / T) / Sd, St, Sd


def test_bounds_after_a_rejection():
    rng = np.random.default_rng(5)
    for _ in range(400):
        V = int(rng.integers(2, 300))
        T = float(np.exp(rng.uniform(np.log(0.05), np.log(5.0))))
        p, q, St, Sd = _rows(rng, V, T, [0.0, 0.01, 0.3, 1.0][rng.integers(4)])
        Z = np.maximum(p - q, 0.0).sum()
        x = int(rng.integers(V))
        assert Z >= q[x] - p[x] - 1e-15
        assert Z >= abs(1.0 / St - 1.0 / Sd) - 1e-15


def test_bounds_on_a_tree_node():
    rng = np.random.default_rng(6)
    for _ in range(300):
        V = int(rng.integers(2, 200))
        T = float(np.exp(rng.uniform(np.log(0.1), np.log(3.0))))
        p, q, St, Sd = _rows(rng, V, T, [0.0, 0.05, 0.5][rng.integers(3)])
        lam, M = 1.0, np.maximum(p - q, 0.0).sum()
        for _ in range(int(rng.integers(1, 6))):
            if M <= 0.0:
                break
            r = np.maximum(p - lam * q, 0.0) / M  # the residual a later child is tested against
            x = int(rng.integers(V))
            nxt = lam + M
            Mn = np.maximum(p - nxt * q, 0.0).sum()
            assert Mn >= M * (q[x] - r[x]) - 1e-14
            assert Mn >= M / Sd - max(0.0, 1.0 / St - lam / Sd) - 1e-14
            assert Mn >= 1.0 / St - nxt / Sd - 1e-14
            lam, M = nxt, Mn
