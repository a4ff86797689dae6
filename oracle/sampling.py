"""fp64 reference for temperature / top-k / top-p sampling over logits.

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing in the HIP
library or its binding may import this module.

Source: the RL.cu pages name sampling among the rollout engine's steps after
the decode and the LM head (pitchhut "Key Features", item 1); they give no
algorithm. This is the usual definition, written out row by row. Readings of
what the pages leave open:

* z = logits / temperature (temperature > 0);
* tokens are ranked by z descending, ties by index ascending; top-k keeps
  the first k of that ranking (1 <= k <= 1024, k > vocab means all);
* top-p applies to the top-k set renormalised (weights w_j = exp(z_j - z_0)
  over the kept ranking, cumulative sums c_j): it keeps the shortest prefix
  whose mass reaches top_p, i.e. ranks 0..cut with cut = min{j : c_j >=
  top_p * c_last}; top_p = 1 keeps the whole top-k set;
* the draw is the inverse CDF in ranking order with the caller's uniform
  u in [0, 1): the token at rank min{j <= cut : c_j > u * c_cut} (strict, so a
  zero-weight token is never drawn). The random number is an input, so the
  result is a deterministic function of (logits, u).
"""
import numpy as np


def ranking(z):
    """Indices of z by value descending, ties by index ascending."""
    return np.lexsort((np.arange(z.shape[0]), -z))


def sample_ref(logits, u, temperature, top_k, top_p):
    """logits [n, V], u [n] -> (tokens [n] int64, cut [n] int64: the number of
    kept ranks minus one, c [n, k] float64: the cumulative weights)."""
    logits = np.asarray(logits, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    n, V = logits.shape
    k = min(int(top_k), V)
    if not (temperature > 0) or k < 1 or not (0 < top_p <= 1):
        raise ValueError("need temperature > 0, top_k >= 1 and 0 < top_p <= 1")
    tokens = np.zeros(n, dtype=np.int64)
    cuts = np.zeros(n, dtype=np.int64)
    cums = np.zeros((n, k))
    for b in range(n):
        z = logits[b] / temperature
        order = ranking(z)[:k]
        w = np.exp(z[order] - z[order[0]])
        c = np.cumsum(w)
        cut = int(min(np.searchsorted(c, top_p * c[-1], side="left"), k - 1))
        j = int(np.searchsorted(c[:cut + 1], u[b] * c[cut], side="right"))
        tokens[b] = order[min(j, cut)]
        cuts[b] = cut
        cums[b] = c
    return tokens, cuts, cums
