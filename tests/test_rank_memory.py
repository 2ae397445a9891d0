"""Per-rank resident model state of stages 1, 2 and 3 against the guide's
memory model (upskillscore guide "ZeRO: particionar estados do treino entre
GPUs", section "Como funciona": 4 Psi + 12 Psi / Nd for P_os, 2 Psi + 14 Psi /
Nd for P_os+g with fp16 gradients, 16 Psi / Nd for P_os+g+p).  Allocation only,
on the CPU: no kernel runs."""
import pytest
import torch

from zero_sharded_mixed_bucketed_amd import rank as zr


@pytest.mark.parametrize("psi,nd", [(1 << 20, 4), (1 << 20, 64), (3 * 5 * 7 * 1024, 15)])
@pytest.mark.parametrize("stage", [1, 2, 3])
def test_resident_bytes_equal_the_model(psi, nd, stage):
    for r in (0, nd - 1):
        st = zr.RankState(psi, nd, r, stage, device=torch.device("cpu"))
        assert st.resident_bytes() == st.model_bytes()


def test_stage2_fp32_gradient_shard_costs_two_more_bytes():
    psi, nd = 1 << 20, 4
    st = zr.RankState(psi, nd, 1, 2, grad_dtype="fp32", device=torch.device("cpu"))
    assert st.resident_bytes() == st.model_bytes() + 2 * psi // nd


def test_stage1_keeps_the_full_local_gradient():
    psi, nd = 1 << 16, 8
    st = zr.RankState(psi, nd, 3, 1, device=torch.device("cpu"))
    assert st.local_grad.numel() == psi
    assert st.grad.data_ptr() == st.local_grad.data_ptr() + 2 * st.geom.offset
    assert st.grad.numel() == st.geom.len


def test_stage3_keeps_only_its_parameter_shard():
    psi, nd = 1 << 16, 8
    st = zr.RankState(psi, nd, 5, 3, device=torch.device("cpu"))
    assert st.param16.numel() == st.geom.len and st.param16_origin == st.geom.offset
    assert st.resident_bytes() == 16 * psi // nd


@pytest.mark.parametrize("kw", [dict(stage=4), dict(stage=0), dict(stage=1, grad_dtype="fp32"),
                                dict(stage=3, grad_dtype="fp32"),
                                dict(stage=2, param_shard=torch.zeros(8, dtype=torch.int16)),
                                dict(stage=3, param_shard=torch.zeros(7, dtype=torch.int16)),
                                dict(stage=2, local_grad=torch.zeros(16, dtype=torch.int16)),
                                dict(stage=1, local_grad=torch.zeros(15, dtype=torch.int16))])
def test_rejects(kw):
    with pytest.raises(ValueError):
        zr.RankState(16, 2, 0, device=torch.device("cpu"), **kw)
