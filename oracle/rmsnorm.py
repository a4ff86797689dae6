"""fp64 reference for RMSNorm forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing in the HIP
library or its binding may import this module.

Source: the RL.cu pages name RMSNorm among the layer operations of the
Qwen3-0.6B stack written in CUDA (pitchhut "Project Highlights"; mlllm.io
"What happened"); they print no formula. RMSNorm is the standard root-mean-
square normalisation, so this is its definition written out, row by row:

  r = 1 / sqrt(mean_j x_j^2 + eps),   y_j = x_j * r * w_j

and its analytic backward for an upstream gradient dy (x_hat = x * r):

  dx_j = r * (w_j dy_j - x_hat_j * mean_k(w_k dy_k x_hat_k)),
  dw_j = sum over rows of dy_j * x_hat_j.

Reading: eps is added to the mean square inside the square root (as in
Qwen3's RMSNorm); the saved per-row statistic is r (the reciprocal RMS).
"""
import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _rrms(x, eps):
    """Reciprocal root mean square of each row of x (eps inside the root)."""
    return 1.0 / np.sqrt((x * x).mean(axis=1) + eps)


def rmsnorm_fwd_ref(x, w, eps):
    """x [rows, n], w [n] -> (y [rows, n], rstd [rows]) in float64."""
    x, w = _f64(x), _f64(w)
    if x.ndim != 2 or w.shape != (x.shape[1],):
        raise ValueError("x must be [rows, n] and w [n]")
    r = _rrms(x, eps)
    return x * r[:, None] * w[None, :], r


def rmsnorm_bwd_ref(x, w, dy, eps):
    """Gradients of sum(y * dy) wrt x and w: (dx [rows, n], dw [n]) float64."""
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    if dy.shape != x.shape:
        raise ValueError("dy must match x")
    r = _rrms(x, eps)
    xh = x * r[:, None]
    g = dy * w[None, :]
    proj = (g * xh).mean(axis=1)
    dx = r[:, None] * (g - xh * proj[:, None])
    dw = (dy * xh).sum(axis=0)
    return dx, dw
