"""Pins of the CPU oracle's building blocks against closed forms, library routines
and a hand-derived case.  None of these re-types the oracle's own formulas: each
expected value comes from mathematics (closed forms, invariances) or from an
independent library routine (scipy, numpy)."""
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

HERE = os.path.dirname(os.path.abspath(__file__))


def bf16(x):
    """Round float values to bfloat16 bit patterns (round to nearest even, torch)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_values(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy().astype(np.float64)


# ------------------------------------------------------------------ softmax / lse

@pytest.mark.parametrize("V,T,c", [(1000, 0.7, 3.25), (7, 1.0, -2.0), (128256, 0.6, 0.0)])
def test_softmax_constant_row_is_uniform(oracle, V, T, c):
    z = np.full(V, c, np.float32)
    lse, p = oracle.softmax_row(z, T)
    assert math.isclose(lse, c / T + math.log(V), rel_tol=0, abs_tol=1e-9)
    assert np.allclose(p, 1.0 / V, rtol=1e-12, atol=0)


@pytest.mark.parametrize("z0,z1,T", [(0.0, 1.0, 1.0), (3.5, -1.25, 0.7), (10.0, 10.0, 2.0), (-4.0, 6.0, 0.3)])
def test_softmax_two_entries_is_logistic(oracle, z0, z1, T):
    lse, p = oracle.softmax_row(np.array([z0, z1], np.float32), T)
    p1 = 1.0 / (1.0 + math.exp(-(z1 - z0) / T))
    assert abs(p[1] - p1) < 1e-14 and abs(p[0] - (1 - p1)) < 1e-14
    assert math.isclose(lse, math.log(math.exp(z0 / T) + math.exp(z1 / T)), rel_tol=1e-14)


def test_softmax_single_entry(oracle):
    lse, p = oracle.softmax_row(np.array([2.5], np.float32), 0.5)
    assert p[0] == 1.0 and math.isclose(lse, 5.0, rel_tol=1e-15)


def test_softmax_shift_invariance(oracle):
    rng = np.random.default_rng(1)
    # a grid of 1/1024 keeps z + 4 exact in fp32 (|z| < 2^12)
    z = (np.round(3 * rng.standard_normal(4096) * 1024) / 1024).astype(np.float32)
    zs = z + np.float32(4.0)
    assert np.array_equal(zs.astype(np.float64), z.astype(np.float64) + 4.0)
    lse0, p0 = oracle.softmax_row(z, 0.8)
    lse1, p1 = oracle.softmax_row(zs, 0.8)
    assert np.allclose(p0, p1, rtol=1e-12, atol=1e-300)
    assert math.isclose(lse1 - lse0, 4.0 / 0.8, rel_tol=0, abs_tol=1e-10)


@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_softmax_matches_scipy(oracle, T):
    rng = np.random.default_rng(7)
    z = (3 * rng.standard_normal(32000)).astype(np.float32)
    lse, p = oracle.softmax_row(z, T)
    zz = z.astype(np.float64) / T
    assert math.isclose(lse, sps.logsumexp(zz), rel_tol=1e-13)
    ref = sps.softmax(zz)
    assert np.allclose(p, ref, rtol=1e-11, atol=0)


def test_bf16_widening_is_exact(oracle):
    # bit patterns: 1.0 = 0x3f80, 2.0 = 0x4000, -inf = 0xff80, 0.5 = 0x3f00
    bits = np.array([0x3F80, 0x4000, 0xFF80, 0x3F00], np.uint16)
    lse, p = oracle.softmax_row(bits, 1.0)
    e = np.exp([1.0, 2.0, 0.5])
    assert p[2] == 0.0
    assert np.allclose(p[[0, 1, 3]], e / e.sum(), rtol=1e-14)
    assert math.isclose(lse, math.log(e.sum()), rel_tol=1e-14)


def test_bf16_matches_torch_rounding(oracle):
    rng = np.random.default_rng(3)
    z = (3 * rng.standard_normal(5000)).astype(np.float32)
    bits = bf16(z)
    vals = bf16_values(bits)
    lse, p = oracle.softmax_row(bits, 0.7)
    assert math.isclose(lse, sps.logsumexp(vals / 0.7), rel_tol=1e-13)


def test_neg_inf_logit_has_zero_probability(oracle):
    z = np.array([0.0, -np.inf, 1.0, -np.inf], np.float32)
    _, p = oracle.softmax_row(z, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    assert math.isclose(p[2], 1 / (1 + math.exp(-1.0)), rel_tol=1e-14)


# ------------------------------------------------------------------ argmax

def test_argmax_matches_numpy_first_occurrence(oracle):
    rng = np.random.default_rng(11)
    for trial in range(200):
        V = int(rng.integers(1, 3000))
        # coarse values make ties frequent
        z = rng.integers(-20, 20, V).astype(np.float32)
        assert oracle.argmax_row(z) == int(np.argmax(z)), trial


def test_argmax_bf16_ties_lowest_index(oracle):
    z = np.zeros(1000, np.float32)
    z[[17, 400, 999]] = 5.0
    assert oracle.argmax_row(bf16(z)) == 17
    assert oracle.argmax_row(bf16(np.full(33, -1.0))) == 0


def test_argmax_with_neg_inf(oracle):
    z = np.array([-np.inf, -np.inf, -3.0, -np.inf], np.float32)
    assert oracle.argmax_row(z) == 2


# ------------------------------------------------------------------ inverse CDF

def _golden():
    rows, draws = {}, []
    with open(os.path.join(HERE, "golden", "dyadic_residual.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "draw":
                draws.append((float(vals[0]), int(vals[1]), float(vals[2])))
            else:
                rows[key] = [float(v) for v in vals]
    return rows, draws


def test_draw_dyadic_golden(oracle):
    rows, draws = _golden()
    p, q = np.array(rows["p"]), np.array(rows["q"])
    w = np.maximum(0.0, p - q)
    assert np.array_equal(w, np.array(rows["w"]))            # dyadic: exact
    assert w.sum() == rows["Z"][0] and np.minimum(p, q).sum() == rows["alpha"][0]
    for u, y, margin in draws:
        got, m = oracle.draw_weights(w, u)
        assert got == y, (u, got, y)
        assert abs(m - margin) < 1e-15, (u, m, margin)


def test_draw_matches_searchsorted(oracle):
    """With positive weights the inverse CDF is numpy's searchsorted(side='right')."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        V = int(rng.integers(1, 500))
        w = rng.random(V) ** 3
        u = float(rng.random())
        c = np.cumsum(w)
        ref = int(np.searchsorted(c, u * c[-1], side="right"))
        got, _ = oracle.draw_weights(w, u)
        if ref < V:
            assert got == ref, trial


def test_draw_never_picks_zero_weight(oracle):
    w = np.array([0.0, 0.0, 0.25, 0.0, 0.75, 0.0])
    for u in np.linspace(0, 0.999999, 101):
        y, _ = oracle.draw_weights(w, float(u))
        assert y in (2, 4)
    # threshold at/after the total (reachable only through rounding): last positive weight
    y, m = oracle.draw_weights(w, 1.0)
    assert y == 4 and m == 0.0
