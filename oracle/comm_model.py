"""Per-step communication volume of plain DP and the three ZeRO-DP stages.

Source: upskillscore guide "ZeRO: particionar estados do treino entre GPUs",
section "Como funciona".  Plain data parallelism moves 2 Psi per step: its
gradient all-reduce is a reduce-scatter followed by an all-gather, each
counted as Psi.  Stage 2 (P_os+g) keeps the same 2 Psi: the gradient
reduce-scatter, then the all-gather of the updated parameters.  Stage 3
(P_os+g+p) needs two parameter all-gathers (one in forward, one in backward)
plus the gradient reduce-scatter: 3 Psi, 1.5x the baseline.  The lastdictionary
entry "ZeRO" adds that stages 1 and 2 keep data parallelism's volume, so stage
1 (P_os) is also one reduce-scatter plus one all-gather.

Readings where the pages are silent:
* Unit: elements of the fp16 parameter/gradient vector; bytes are 2 per
  element.
* The pages' count charges each collective Psi.  A bandwidth-optimal
  reduce-scatter or all-gather over Nd ranks (ring or direct) makes each rank
  send (Nd - 1) / Nd of the vector, so the exact per-rank send volume is
  collectives x Psi x (Nd - 1) / Nd; it tends to the pages' count as Nd grows
  and is 0 for Nd = 1 (nothing to exchange).  Both are returned.

Pins (tests/test_oracle_comm_model.py): the guide's 2 Psi / 2 Psi / 3 Psi and
the ratio 1.5; stage 1 equal to plain DP (dictionary entry); the exact form's
limit and its Nd = 1 and Nd = 2 values, counted by brute force over the chunks
a ring reduce-scatter and all-gather send.
"""
from __future__ import annotations

from dataclasses import dataclass

FP16_BYTES = 2

# (reduce-scatters, all-gathers) per step, in the order the step issues them
_COLLECTIVES = {
    0: ("reduce_scatter", "all_gather"),                # gradient all-reduce
    1: ("reduce_scatter", "all_gather"),                # grads to owners, params back
    2: ("reduce_scatter", "all_gather"),
    3: ("all_gather", "all_gather", "reduce_scatter"),  # params fwd, params bwd, grads
}


@dataclass(frozen=True)
class Comm:
    collectives: tuple
    elems: float                # the pages' count: Psi per collective
    elems_sent_per_rank: float  # bandwidth-optimal collectives: (Nd - 1) / Nd of Psi each

    @property
    def bytes_sent_per_rank(self) -> float:
        return FP16_BYTES * self.elems_sent_per_rank


def comm_volume(psi: float, nd: int, stage: int) -> Comm:
    if nd < 1:
        raise ValueError("nd must be >= 1")
    if stage not in _COLLECTIVES:
        raise ValueError("stage must be 0 (DP), 1, 2 or 3")
    cs = _COLLECTIVES[stage]
    return Comm(cs, len(cs) * psi, len(cs) * psi * (nd - 1) / nd)
