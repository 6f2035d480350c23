"""fp64 oracle for the wide-row reduction-reuse workloads (softmax over
logits, LayerNorm).

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.  It shares no code
with the HIP library and imports nothing from it.

Source: the CREDIT summary, section III.B "Reduction-Reuse Transformation"
(a row's elements are reduced to scalar statistics, then an elementwise
function of each element and the statistics gives every output element) and
section V.A "Experimental Setup" (FP32 workloads, LayerNorm and softmax-logits
among them, row widths 4K to 64K, 2048 LayerNorm rows and 4096 rows for the
others).  The pages give neither formula; the readings are the standard
definitions:

* softmax over a row x of width W:  y_i = exp(x_i - m) / sum_j exp(x_j - m),
  m = max_j x_j  (the subtraction leaves y unchanged and keeps exp finite);
* LayerNorm over a row:  mu = sum_j x_j / W,  var = sum_j (x_j - mu)^2 / W
  (biased), y_i = (x_i - mu) / sqrt(var + eps) * gamma_i + beta_i, with
  per-column gamma and beta and eps = 1e-5.

Inputs are float32 arrays; they are widened exactly to float64 and every step
below runs in float64, one row at a time, in the order the definitions give:
first the statistics, then the elementwise function.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-5


def softmax_rows(x: np.ndarray) -> np.ndarray:
    """[M][W] float32 -> [M][W] float64 softmax of each row."""
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("softmax_rows needs a [rows][width >= 1] array")
    out = np.empty(x.shape, dtype=np.float64)
    for r in range(x.shape[0]):
        row = x[r].astype(np.float64)
        m = row.max()                         # statistic 1: the row maximum
        e = np.exp(row - m)
        s = e.sum()                           # statistic 2: the sum of exponentials
        out[r] = e / s                        # elementwise function of x_i, m, s
    return out


def layernorm_rows(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = EPS) -> np.ndarray:
    """[M][W] float32 rows, [W] gamma and beta -> [M][W] float64 LayerNorm."""
    x = np.asarray(x)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("layernorm_rows needs a [rows][width >= 1] array")
    W = x.shape[1]
    g = np.asarray(gamma, dtype=np.float64).reshape(W)
    b = np.asarray(beta, dtype=np.float64).reshape(W)
    out = np.empty(x.shape, dtype=np.float64)
    for r in range(x.shape[0]):
        row = x[r].astype(np.float64)
        mu = row.sum() / W                    # statistic 1: the mean
        var = ((row - mu) ** 2).sum() / W     # statistic 2: the biased variance
        out[r] = (row - mu) / np.sqrt(var + eps) * g + b
    return out
