"""fp64 references for the other streaming reductions (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and bench's ``cpu_baseline``;
never by the product path, and it imports nothing from it.

The math-properties page, section 8 ("Generalization"), lists operations
with the same structure as attention's softmax -- softmax-based routing,
mixture-of-experts gating, LayerNorm and GroupNorm -- as convertible into a
streaming reduction (its section 2: a finite state updated block by block).
The pages give no formulas for them; the operations are their usual
definitions, written out here in two passes:

* Row softmax (routing / gating scores): y_j = exp(x_j - m) / l with
  m = max_j x_j, l = sum_j exp(x_j - m), and lse = m + ln l.  A row whose
  entries are all -inf has y = 0 and lse = -inf (the attention convention).
* LayerNorm over a row of n values: mean = sum x / n, var = sum (x - mean)^2 / n
  (population variance), rstd = 1 / sqrt(var + eps),
  y_e = (x_e - mean) * rstd * gamma[c] + beta[c].
  GroupNorm is the same over rows that are the groups of a sample: for an
  input [N, C, S] with G groups, row r = (sample, group g) holds the C/G
  channels of group g, each of S values; element e of the row belongs to
  channel c = g * (C/G) + e // S.  LayerNorm is G = 1, S = 1 (c = e).

The streaming states these reductions carry (what the kernels merge), for the
pins:

* softmax: (m, l), merged by the merge equation of the FlashAttention summary
  page (section "Incremental softmax tracking"): ``streaming.merge_stats``.
* moments: (n, mean, M2) with M2 = sum (x - mean)^2, merged by the pairwise
  update of Chan, Golub and LeVeque ("Updating formulae and a pairwise
  algorithm for computing sample variances", 1979):
      n = na + nb, delta = mean_b - mean_a,
      mean = mean_a + delta * nb / n, M2 = M2_a + M2_b + delta^2 na nb / n.
"""
from __future__ import annotations

import numpy as np

__all__ = ["softmax_rows", "layernorm_rows", "affine_index", "merge_moments", "streaming_moments"]


def softmax_rows(x):
    """Row softmax of a 2-D array (fp64).  Returns (y [R, L], lse [R])."""
    x = np.asarray(x, np.float64)
    valid = ~np.all(np.isneginf(x), axis=1)
    m = np.where(valid, np.max(x, axis=1), 0.0)
    e = np.where(np.isneginf(x), 0.0, np.exp(x - m[:, None]))
    l = e.sum(axis=1)
    y = np.where(valid[:, None], e / np.where(valid, l, 1.0)[:, None], 0.0)
    lse = np.where(valid, m + np.log(np.where(valid, l, 1.0)), -np.inf)
    return y, lse


def affine_index(rows, cols, groups=1, inner=1):
    """Channel index [R, L] of each element for the affine step (see module doc)."""
    r = np.arange(rows, dtype=np.int64)[:, None]
    e = np.arange(cols, dtype=np.int64)[None, :]
    cpg = cols // inner
    return (r % groups) * cpg + e // inner


def layernorm_rows(x, gamma=None, beta=None, eps=1e-5, groups=1, inner=1):
    """LayerNorm / GroupNorm of each row (fp64).  Returns (y, mean [R], rstd [R]).

    gamma, beta: 1-D arrays of groups * cols // inner channels, or None
    (scale 1, shift 0)."""
    x = np.asarray(x, np.float64)
    R, L = x.shape
    mean = x.sum(axis=1) / L
    var = ((x - mean[:, None]) ** 2).sum(axis=1) / L
    rstd = 1.0 / np.sqrt(var + float(eps))
    y = (x - mean[:, None]) * rstd[:, None]
    idx = affine_index(R, L, groups, inner)
    if gamma is not None:
        y = y * np.asarray(gamma, np.float64)[idx]
    if beta is not None:
        y = y + np.asarray(beta, np.float64)[idx]
    return y, mean, rstd


def merge_moments(a, b):
    """Chan-Golub-LeVeque merge of two (n, mean, M2) states (arrays allowed)."""
    na, ma, m2a = a
    nb, mb, m2b = b
    n = na + nb
    safe = np.where(n > 0, n, 1)
    delta = mb - ma
    mean = np.where(n > 0, ma + delta * nb / safe, 0.0)
    m2 = m2a + m2b + delta * delta * na * nb / safe
    return n, mean, m2


def streaming_moments(x, blocks):
    """(n, mean, M2) of a 1-D array, visiting the index blocks in order and
    merging each block's own two-pass moments into the running state."""
    x = np.asarray(x, np.float64)
    state = (0, 0.0, 0.0)
    for idx in blocks:
        v = x[np.asarray(idx, dtype=np.int64)]
        if v.size == 0:
            continue
        mb = v.mean()
        state = merge_moments(state, (v.size, mb, float(((v - mb) ** 2).sum())))
    return state
