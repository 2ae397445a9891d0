"""Stage 3 (P_os+g+p): the parameters are partitioned as well, and each
layer's full fp16 parameters are gathered just in time, used and released.

Sources:
* upskillscore guide "ZeRO: particionar estados do treino entre GPUs", section
  "Como funciona": in the third stage the parameters are partitioned too and a
  process that needs another's partition receives it; memory falls to
  16 Psi / Nd; communication is two parameter all-gathers (forward and
  backward) plus the gradient reduce-scatter.
* lastdictionary entry "ZeRO": in stage 3 a layer's parameters are fetched
  right before that layer runs and dropped once it is done.
* llm-engineer card "ZeRO-2", section "Why all-gather is still needed": the
  all-gather of the rank partitions, in rank order, is the full vector
  [A, B, C].

What one rank computes, written from those passages:
* gather_params -- the receive side of one layer's all-gather: the fp16
  parameters of flat range [lo, lo + n), where flat index i lives in rank
  i // S's shard at position i - (i // S) * S (contiguous rank-major shards of
  S = ceil(Psi / Nd), as for stages 1 and 2);
* the rest of a stage-3 step reuses the stage-2 pieces: each layer's gradient
  is reduced into the rank's gradient shard (oracle.reduce) and the Adam step
  (oracle.adam) writes the rank's own fp16 parameter shard, which is what the
  next step's gathers read.

Pins (tests/test_oracle_stage3.py): the gathers of every layer, concatenated,
rebuild the concatenation of the shards (the [A, B, C] of the card); each
gathered element equals the one found by scanning every rank's owned range
(brute force on tiny models, ragged last shards, layers crossing several
shards); the per-device bytes of a stage-3 rank equal 16 Psi / Nd.
"""
from __future__ import annotations

import numpy as np

from . import geometry


def gather_params(shards: np.ndarray, psi: int, nd: int, lo: int, n: int) -> np.ndarray:
    """shards: uint16 [Nd, >= S], row k = rank k's fp16 parameter shard.
    Returns uint16 [n]: the parameters of flat [lo, lo + n)."""
    if lo < 0 or n < 0 or lo + n > psi:
        raise ValueError("range beyond the parameter vector")
    s = geometry.shard_size(psi, nd)
    i = np.arange(lo, lo + n, dtype=np.int64)
    k = i // s
    return shards[k, i - k * s]
