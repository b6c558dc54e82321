"""Split-context partial states and their log-sum-exp merge, in float64.

TEST INFRASTRUCTURE ONLY (part of the CPU oracle; see the package header).

The ROCm blog "Optimizing ATOM and vLLM-ATOM for High-Interactivity
Inference" ("Attention Decode: Split Memory Work to Fill the Device")
describes decode attention that splits the KV range of a sequence into
several pieces so that a single query fills the device, keeps one
log-sum-exp value per split in float32, and merges the splits afterwards.
The page gives no formulas; the steps below are the plain reading:

* a split over keys ``J`` with logits ``x_j`` and values ``v_j`` summarises
  itself as ``m = max_j x_j``, ``l = sum_j exp(x_j - m)`` and the normalised
  partial output ``o = sum_j exp(x_j - m) v_j / l`` (an empty split has
  ``m = -inf``, ``l = 0`` and contributes nothing);
* the merge forms ``lse_p = m_p + ln l_p``, ``M = max_p lse_p`` and returns
  ``sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M)``.

Merging the splits of any partition of the keys equals softmax attention over
all keys (the tests check this); the GPU reduce follows the same formula in
base 2.
"""
from __future__ import annotations

import numpy as np

__all__ = ["partial_state", "merge_states"]


def partial_state(x, v):
    """Summary (m, l, o) of one split: logits ``x`` ``[J]``, values ``v`` ``[J, D]``."""
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if x.size == 0:
        return -np.inf, 0.0, np.zeros(v.shape[-1])
    m = x.max()
    e = np.exp(x - m)
    l = e.sum()
    return m, l, (e @ v) / l


def merge_states(states):
    """Log-sum-exp merge of split summaries ``[(m, l, o), ...]``."""
    lse = np.array([m + np.log(l) if l > 0 else -np.inf for m, l, _ in states])
    M = lse.max()
    w = np.exp(lse - M)
    o = np.stack([st[2] for st in states])
    return (w[:, None] * o).sum(axis=0) / w.sum()
