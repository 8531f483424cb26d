"""Plain fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The HIP library and its Python binding never import it, and it imports nothing
from them.

* :mod:`oracle.attention` -- the plain definition (two passes over full score
  rows) of the forward output, the log-sum-exp statistics and the analytic
  gradients.
* :mod:`oracle.streaming` -- the pages' block-by-block recurrence (running max,
  running sum, rescaled output), used only to pin the definition against the
  method's own algorithm.
* :mod:`oracle.dropout` -- the Philox4x32-10 generator and the dropout keep
  mask (used through the ``dropout=`` argument of the attention functions).
* :mod:`oracle.reductions` -- row softmax and LayerNorm / GroupNorm, the other
  streaming reductions, plus the moment merge used to pin them.
"""
from .attention import (allowed_mask, forward, backward, forward_rows,
                        gradients_sampled, probabilities)
from .streaming import merge_stats, streaming_forward
from .dropout import keep_mask, keep_scale, drop_threshold, philox4x32_10
from .reductions import softmax_rows, layernorm_rows, merge_moments, streaming_moments

__all__ = ["allowed_mask", "forward", "backward", "forward_rows",
           "probabilities", "gradients_sampled", "merge_stats", "streaming_forward",
           "keep_mask", "keep_scale", "drop_threshold", "philox4x32_10",
           "softmax_rows", "layernorm_rows", "merge_moments", "streaming_moments"]
