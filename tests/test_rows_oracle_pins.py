"""Pins for the fp64 row oracle (softmax over logits, LayerNorm), against facts
that do not come from the oracle: closed forms, invariances the definitions
fix, library special cases and 50-digit brute force.  Each pin is chosen so a
plausible slip fails it: a missing max subtraction (overflow at large
logits), the wrong axis, unbiased instead of biased variance, eps outside the
square root, gamma/beta indexed by row instead of column."""
import math

import numpy as np
import pytest

from oracle import rows_np


def test_softmax_uniform_row():
    for W in (1, 7, 4096):
        y = rows_np.softmax_rows(np.full((2, W), 3.25, np.float32))
        assert np.all(y == 1.0 / W) or np.max(np.abs(y - 1.0 / W)) <= 1e-18


def test_softmax_two_logits_is_logistic():
    for a in (-7.0, -0.5, 0.0, 2.0, 30.0):
        y = rows_np.softmax_rows(np.array([[a, 0.0]], np.float32))
        s, t = 1.0 / (1.0 + math.exp(-a)), 1.0 / (1.0 + math.exp(a))    # t = 1 - s without cancellation
        assert abs(y[0, 0] - s) <= 4e-16 * s and abs(y[0, 1] - t) <= 4e-16 * t


def test_softmax_large_logits_and_shift():
    x = np.array([[1000.0, 999.0, -1000.0], [0.0, -1.0, -2000.0]], np.float32)
    y = rows_np.softmax_rows(x)
    assert np.all(np.isfinite(y))
    # both rows hold the same differences up to the last entry's underflow
    np.testing.assert_allclose(y[0, :2], y[1, :2], rtol=0, atol=1e-16)
    e = 1.0 / (1.0 + math.exp(-1.0))
    assert abs(y[0, 0] - e) <= 1e-16


def test_softmax_rows_are_independent():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 5)).astype(np.float32)
    y = rows_np.softmax_rows(x)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    y0 = rows_np.softmax_rows(x[1:2])
    assert np.array_equal(y[1], y0[0])


def test_layernorm_constant_row_gives_beta():
    W = 33
    g = np.linspace(0.5, 2.0, W).astype(np.float32)
    b = np.linspace(-1.0, 1.0, W).astype(np.float32)
    y = rows_np.layernorm_rows(np.full((2, W), -4.5, np.float32), g, b)
    assert np.array_equal(y, np.tile(b.astype(np.float64), (2, 1)))


@pytest.mark.parametrize("a,b", [(3.0, -1.0), (0.001, 0.003), (10.0, 10.0)])
def test_layernorm_two_columns_closed_form(a, b):
    # mu = (a + b) / 2, biased var = ((a - b) / 2)^2, eps inside the root
    g = np.array([1.5, -0.5], np.float32)
    be = np.array([0.25, 2.0], np.float32)
    x = np.array([[a, b]], np.float32)
    a, b = float(x[0, 0]), float(x[0, 1])
    h = (a - b) / 2.0
    r = 1.0 / math.sqrt(h * h + rows_np.EPS)
    want = [h * r * float(g[0]) + float(be[0]), -h * r * float(g[1]) + float(be[1])]
    y = rows_np.layernorm_rows(x, g, be)
    np.testing.assert_allclose(y[0], want, rtol=1e-15, atol=1e-15)


def test_layernorm_moments_and_column_parameters():
    rng = np.random.default_rng(1)
    M, W = 3, 257
    x = (rng.standard_normal((M, W)) * 5 + 2).astype(np.float32)
    y = rows_np.layernorm_rows(x, np.ones(W, np.float32), np.zeros(W, np.float32), eps=0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y ** 2).mean(axis=1), 1.0, rtol=1e-13)
    # gamma, beta act per column, the same for every row
    g = rng.standard_normal(W).astype(np.float32)
    b = rng.standard_normal(W).astype(np.float32)
    y2 = rows_np.layernorm_rows(x, g, b, eps=0.0)
    np.testing.assert_allclose(y2, y * g.astype(np.float64) + b.astype(np.float64), rtol=1e-13, atol=1e-13)


def test_library_special_cases():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 300)).astype(np.float32)
    g = rng.standard_normal(300).astype(np.float32)
    b = rng.standard_normal(300).astype(np.float32)
    xt = torch.from_numpy(x).double()
    ref_sm = torch.softmax(xt, dim=1).numpy()
    ref_ln = torch.nn.functional.layer_norm(xt, (300,), torch.from_numpy(g).double(),
                                            torch.from_numpy(b).double(), eps=rows_np.EPS).numpy()
    np.testing.assert_allclose(rows_np.softmax_rows(x), ref_sm, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(rows_np.layernorm_rows(x, g, b), ref_ln, rtol=1e-12, atol=1e-13)


def test_brute_force_mpmath():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 9)) * 3).astype(np.float32)
    g = rng.standard_normal(9).astype(np.float32)
    b = rng.standard_normal(9).astype(np.float32)
    sm = rows_np.softmax_rows(x)
    ln = rows_np.layernorm_rows(x, g, b)
    for r in range(2):
        xs = [mp.mpf(float(v)) for v in x[r]]
        es = [mp.e ** v for v in xs]
        tot = mp.fsum(es)
        for i in range(9):
            want = float(es[i] / tot)
            assert abs(want - sm[r, i]) <= 4e-16 * want
        mu = mp.fsum(xs) / 9
        var = mp.fsum((v - mu) ** 2 for v in xs) / 9
        rs = 1 / mp.sqrt(var + mp.mpf(rows_np.EPS))
        for i in range(9):
            want = (xs[i] - mu) * rs * mp.mpf(float(g[i])) + mp.mpf(float(b[i]))
            assert abs(float(want) - ln[r, i]) <= 1e-14 * max(1.0, abs(float(want)))


def test_rejects_empty_rows():
    with pytest.raises(ValueError):
        rows_np.softmax_rows(np.zeros((2, 0), np.float32))
    with pytest.raises(ValueError):
        rows_np.layernorm_rows(np.zeros((0,), np.float32), np.zeros(0), np.zeros(0))
