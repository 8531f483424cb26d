"""Dropout keep mask for the fp64 oracle (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` (and through the oracle by
``__graft_entry__.smoke()`` / bench's ``cpu_baseline``); never by the product
path, and it imports nothing from it.

The FlashAttention summary page (paper 2205.14135), section "Key ideas",
kernel-fusion bullet, names dropout among the steps fused into the kernel but
fixes nothing about it.  The contract written here (and implemented
independently on the GPU) is:

* Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
  Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): a
  four-word counter and a two-word key, ten rounds, each round
      (c0, c1, c2, c3) <- (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
  with the 32x32 -> 64-bit products split into high and low words, and the key
  bumped by the Weyl constants (W0, W1) after every round but the last.
* Mapping: the (query i, key j) plane of head bh = b*H + h is cut into 4x4
  blocks.  Block (i // 4, j // 4) is the counter (i // 4, j // 4, bh, offset)
  under the key (seed mod 2^32, seed div 2^32); output word w holds the
  decisions of query 4 (i // 4) + w, its byte k (bits 8k..8k+7) the decision
  of key 4 (j // 4) + k.
* Decision: the drop probability p is rounded to t / 256 with
  t = round(256 p) clamped to [0, 255]; key j is kept for query i iff its
  byte >= t.  Kept probabilities are scaled by 1 / (1 - t/256), so E[Z] = 1.
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "drop_threshold", "keep_scale", "keep_mask"]

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on arrays of counters (broadcast together) and one key.

    Returns the four output words as uint64 arrays holding 32-bit values.
    """
    c = [np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3)]
    c = list(np.broadcast_arrays(*c))
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for r in range(10):
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        if r < 9:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
    return c


def drop_threshold(p):
    """Byte threshold t: a decision byte below t drops the element."""
    if not (0.0 <= float(p) < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(min(255, max(0, round(float(p) * 256.0))))


def keep_scale(p):
    """Scale 1 / (1 - t / 256) applied to kept probabilities."""
    return 256.0 / (256.0 - drop_threshold(p))


def keep_mask(bh, rows, cols, p, seed, offset=0):
    """Boolean [len(rows), len(cols)]: True where key cols[c] is kept for
    query rows[r] in head bh (see the module docstring for the mapping)."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    cols = np.asarray(cols, dtype=np.int64).reshape(-1)
    t = drop_threshold(p)
    seed = int(seed)
    # one generator call per distinct 4x4 block, then each element picks its
    # word (query) and byte (key) out of its block's output
    qblk, qidx = np.unique(rows // 4, return_inverse=True)
    kblk, kidx = np.unique(cols // 4, return_inverse=True)
    words = np.stack(philox4x32_10(qblk[:, None], kblk[None, :], int(bh), int(offset) & 0xFFFFFFFF,
                                   seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    word = words[(rows % 4)[:, None], qidx.reshape(-1)[:, None], kidx.reshape(-1)[None, :]]
    byte = (word >> (np.uint64(8) * (cols % 4).astype(np.uint64))[None, :]) & np.uint64(0xFF)
    return byte >= np.uint64(t)
