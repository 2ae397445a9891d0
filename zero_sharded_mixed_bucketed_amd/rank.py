"""One data-parallel rank's model-state buffers for ZeRO stages 1, 2 and 3,
and the steps over them through the C ABI.

What a rank keeps (upskillscore guide "ZeRO: particionar estados do treino
entre GPUs", section "Como funciona", with its 2 Psi / 2 Psi / 12 Psi
accounting; llm-engineer card "ZeRO-2", sections "ZeRO-1's remaining waste"
and "Gradient lifecycle"):

* both stages: the flat fp16 parameter vector [Psi] (the all-gather target;
  the rank writes its slot) and the fp32 master/m/v of its shard [S];
* stage 1 (P_os): its full fp16 local gradient [Psi], kept for the whole
  backward pass; the reduced gradient of the owned slice is written in place
  into that buffer's slot [offset, offset + S) -- 4 Psi + 12 Psi / Nd bytes;
* stage 2 (P_os+g): only a gradient shard [S], fp16 (the guide's accounting,
  2 Psi + 14 Psi / Nd bytes) or fp32; each bucket's local gradient is
  released once its owner has reduced it.
* stage 3 (P_os+g+p; lastdictionary entry "ZeRO"): the parameters are
  partitioned too.  The rank keeps its fp16 parameter shard [S] instead of the
  flat vector (16 Psi / Nd bytes in all).  Each layer's parameters are gathered
  from the rank shards just in time (gather_layer) and released after use.

This module allocates with torch and calls the library; no arithmetic of the
path happens here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import adam_step_shard, gather_params, memory_model, reduce_shard, shard_geometry

STAGE_OS = 1
STAGE_OS_G = 2
STAGE_OS_G_P = 3


class RankState:
    """Device buffers of rank `rank` of `nd` over a `psi`-parameter model.

    grad_dtype is the gradient the reduce writes and Adam reads: "fp16" (the
    pages' accounting) or, for stage 2 only, "fp32".  local_grad (stage 1
    only): an existing contiguous [psi] fp16 buffer to keep as the local
    gradient, e.g. row `rank` of a buffer that holds every rank's local
    gradient when all ranks are simulated on one device.  param_shard (stage 3
    only): likewise, an existing contiguous [S] fp16 buffer to keep as the
    rank's parameter shard.
    """

    def __init__(self, psi: int, nd: int, rank: int, stage: int, grad_dtype: str = "fp16",
                 device: Optional[torch.device] = None, local_grad=None, param_shard=None):
        if stage not in (STAGE_OS, STAGE_OS_G, STAGE_OS_G_P):
            raise ValueError("stage must be 1 (P_os), 2 (P_os+g) or 3 (P_os+g+p)")
        if grad_dtype not in ("fp16", "fp32") or (stage != STAGE_OS_G and grad_dtype != "fp16"):
            raise ValueError("grad_dtype: fp16, or fp32 for stage 2")
        dev = device or torch.device("cuda", torch.cuda.current_device())
        self.stage, self.grad_dtype = stage, grad_dtype
        self.geom = shard_geometry(psi, nd, rank)
        s = self.geom.len
        if stage == STAGE_OS_G_P:
            if param_shard is None:
                param_shard = torch.zeros(s, dtype=torch.int16, device=dev)
            elif (param_shard.dtype not in (torch.int16, torch.float16) or param_shard.dim() != 1
                  or param_shard.numel() != s or not param_shard.is_contiguous()):
                raise ValueError("param_shard must be a contiguous [S] fp16 buffer")
            self.param16 = param_shard                # window origin: the shard's offset
            self.param16_origin = self.geom.offset
        else:
            if param_shard is not None:
                raise ValueError("param_shard is for stage 3")
            self.param16 = torch.zeros(psi, dtype=torch.int16, device=dev)
            self.param16_origin = 0
        self.master = torch.zeros(s, dtype=torch.float32, device=dev)
        self.m = torch.zeros(s, dtype=torch.float32, device=dev)
        self.v = torch.zeros(s, dtype=torch.float32, device=dev)
        lo = self.geom.offset
        if stage == STAGE_OS:
            if local_grad is None:
                local_grad = torch.zeros(psi, dtype=torch.int16, device=dev)
            elif (local_grad.dtype not in (torch.int16, torch.float16) or local_grad.dim() != 1
                  or local_grad.numel() != psi or not local_grad.is_contiguous()):
                raise ValueError("local_grad must be a contiguous [psi] fp16 buffer")
            self.local_grad = local_grad
            self.grad = self.local_grad[lo:lo + s]          # the reduced slice, in place
        else:
            if local_grad is not None:
                raise ValueError("local_grad is for stage 1")
            self.local_grad = None
            dt = torch.int16 if grad_dtype == "fp16" else torch.float32
            self.grad = torch.zeros(s, dtype=dt, device=dev)

    def resident_tensors(self):
        """The buffers this rank keeps across the step (views not counted twice)."""
        ts = [self.param16, self.master, self.m, self.v]
        ts.append(self.local_grad if self.stage == STAGE_OS else self.grad)
        return ts

    def resident_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in self.resident_tensors())

    def model_bytes(self) -> float:
        """The guide's per-device bytes for this stage (fp16 gradients)."""
        return memory_model(self.geom.psi, self.geom.nd, self.stage)

    def reduce_bucket(self, bucket_offset: int, bucket_len: int, slices, stream=None) -> None:
        """The owner's reduce of one bucket: slices are the Nd ranks' local
        gradients over [bucket_offset, bucket_offset + bucket_len), one row each.
        In stage 1 row `rank` may be this rank's own local_grad (aliasing it
        column for column is allowed)."""
        if self.grad.dtype == torch.float32:
            reduce_shard(self.geom, bucket_offset, bucket_len, slices, self.grad, None,
                         stream=stream)
        else:
            reduce_shard(self.geom, bucket_offset, bucket_len, slices, None, self.grad,
                         stream=stream)

    def adam_step(self, lr: float, beta1: float, beta2: float, eps: float, step: int,
                  stream=None) -> None:
        adam_step_shard(self.geom, self.master, self.m, self.v, self.grad, self.param16,
                        self.param16_origin, lr, beta1, beta2, eps, step, stream=stream)

    def gather_layer(self, lo: int, length: int, shards, out, stream=None) -> None:
        """Stage 3: the parameters of flat [lo, lo + length) into `out`, from the
        rank shards [Nd, >= S] (row `rank` is this rank's param16 when all ranks
        are simulated on one device)."""
        if self.stage != STAGE_OS_G_P:
            raise ValueError("only stage 3 gathers parameters")
        gather_params(self.geom.psi, self.geom.nd, lo, length, shards, out, stream=stream)
