"""The pages' block-by-block recurrence, in fp64 (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and nothing in the product).
It exists to pin :mod:`oracle.attention` against the method's own algorithm:
in exact arithmetic both give the same O and statistics.

* FlashAttention summary page, section "Incremental softmax tracking", the
  merge equation: for a vector split into two parts, the maximum is the larger
  of the two maxima and the exponential sum is each part's sum rescaled by
  exp(part max - total max), then added.  :func:`merge_stats`.
* Same section, the four numbered per-block steps for query block i and
  key/value block j: scores of the block; the block's own row max, exp and
  row sum; the running max/sum update; the running output update, which
  rescales the previous output by l_old * exp(m_old - m_new), adds
  exp(m_block - m_new) times the block's exp-scores times V_j, and divides by
  the new sum.  :func:`streaming_forward` follows these steps in that order,
  including the division at every step.
* Math-properties page, section 7 (stateful streaming): the state carried
  across key/value blocks is the running max, the exponential sum and the
  partial output.
"""
from __future__ import annotations

import numpy as np

__all__ = ["merge_stats", "streaming_forward"]


def merge_stats(m1, l1, m2, l2):
    """Combine (max, exp-sum) statistics of two parts of the same row(s).

    Parts with no visible entry carry m = -inf and l = 0.
    """
    m1 = np.asarray(m1, np.float64)
    m2 = np.asarray(m2, np.float64)
    m = np.maximum(m1, m2)
    safe = np.where(np.isfinite(m), m, 0.0)
    l = np.exp(m1 - safe) * l1 + np.exp(m2 - safe) * l2
    return m, l


def streaming_forward(q, k, v, scale, key_blocks, *, allowed=None):
    """One (batch, head), one query block, processed over a list of key blocks.

    q: [R, d]; k, v: [N, d]; key_blocks: list of index arrays partitioning
    (a subset of) range(N); ``allowed``: optional boolean [R, N] mask.
    Returns (o [R, d], m [R], l [R]) after the last block.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    R, d = q.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    o = np.zeros((R, d))
    for cols in key_blocks:
        cols = np.asarray(cols, dtype=np.int64)
        # step 1: block scores
        s = float(scale) * (q @ k[cols].T)
        if allowed is not None:
            s = np.where(allowed[:, cols], s, -np.inf)
        # step 2: block-local max, exp-scores and row sum
        m_blk = np.max(s, axis=1) if cols.size else np.full(R, -np.inf)
        m_blk_safe = np.where(np.isfinite(m_blk), m_blk, 0.0)
        p_blk = np.exp(s - m_blk_safe[:, None])
        l_blk = p_blk.sum(axis=1)
        # step 3: running statistics
        m_new, l_new = merge_stats(m, l, m_blk, l_blk)
        m_new_safe = np.where(np.isfinite(m_new), m_new, 0.0)
        # step 4: running (normalised) output
        a_old = l * np.exp(m - m_new_safe)
        a_blk = np.exp(m_blk - m_new_safe)
        num = a_old[:, None] * o + a_blk[:, None] * (p_blk @ v[cols])
        o = np.where(l_new[:, None] > 0, num / np.where(l_new > 0, l_new, 1.0)[:, None], 0.0)
        m, l = m_new, l_new
    return o, m, l
