"""CPU oracle of the per-rank ZeRO stage-1/2 path -- TEST INFRASTRUCTURE.

A plain, slow, obviously correct NumPy implementation of what the GPU path
computes, written from the pages on ZeRO (the upskillscore guide "ZeRO:
particionar estados do treino entre GPUs", the lastdictionary entry "ZeRO",
and the llm-engineer card "ZeRO-2").  Only the tests, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py`` may import it.  The product path never
does, and this package imports nothing from the product (no HIP library, no
torch): the two share only the seeded input generators in ``synth``.

Modules:
  memory_model -- per-device model-state bytes of plain DP and ZeRO stages 1-3
  comm_model   -- per-step communication volume of plain DP and ZeRO stages 1-3
  geometry     -- contiguous rank-major shards, bucket/shard intersections
  reduce       -- the owner's reduce-scatter slice of one gradient bucket
  adam         -- the sharded mixed-precision Adam step and the fp16 slot write
  stage3       -- the receive side of a stage-3 layer parameter gather

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (printed values, closed forms, brute force, an fp64 textbook
shadow); see each module's header for the pins.
"""
from . import adam, comm_model, geometry, memory_model, reduce, stage3  # noqa: F401
