"""Host-side checks of the Python binding: arguments are validated (device
residency, contiguity, dtypes, packed offsets) before any pointer reaches the
library. CPU tensors suffice: every case raises before a launch."""
import pytest
import torch

import delta_rule_linear_gdr_amd as gdr


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def _args(B=1, T=64, H=2, dk=128, dv=128, vec=False):
    q, k = _t(B, T, H, dk), _t(B, T, H, dk)
    v = _t(B, T, H, dv)
    g = _t(B, T, H, dk, dtype=torch.float32) if vec else _t(B, T, H, dtype=torch.float32)
    beta = _t(B, T, H)
    return q, k, v, g, beta


def test_host_tensors_are_refused():
    with pytest.raises(ValueError, match="device tensor"):
        gdr.gdr_fwd(*_args())


def test_dtype_mismatch_is_refused(monkeypatch):
    # pretend the tensors are on the device so that the dtype checks run
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))
    q, k, v, g, beta = _args()
    with pytest.raises(TypeError, match="differs from q dtype"):
        gdr.gdr_fwd(q, k.float(), v, g, beta)
    with pytest.raises(TypeError, match="float32"):
        gdr.gdr_fwd(q, k, v, g.to(torch.bfloat16), beta)


def test_noncontiguous_is_refused(monkeypatch):
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))
    q, k, v, g, beta = _args()
    with pytest.raises(ValueError, match="contiguous"):
        gdr.gdr_fwd(q.transpose(1, 2), k, v, g, beta)


def test_packed_offsets_are_checked(monkeypatch):
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))
    q, k, v, g, beta = _args()
    with pytest.raises(ValueError, match="int64"):
        gdr.gdr_fwd(q, k, v, g, beta, cu_seqlens=torch.tensor([0, 64], dtype=torch.int32))
    with pytest.raises(ValueError, match="batch size 1"):
        gdr.gdr_fwd(*_args(B=2), cu_seqlens=torch.tensor([0, 64], dtype=torch.int64))
    with pytest.raises(ValueError):
        gdr.gdr_fwd(q, k, v, g, beta, cu_seqlens=torch.zeros(0, dtype=torch.int64))


def test_descriptor_follows_the_tensors():
    q, k, v, g, beta = _args(dk=80, dv=112, vec=True)
    d = gdr._desc_from(q, g, v)
    assert (d.DK, d.DV, d.gate, d.dtype) == (80, 112, gdr.GATE_VECTOR, gdr.DT_BF16)
    d = gdr._desc_from(q.float(), None, v)
    assert (d.gate, d.dtype) == (gdr.GATE_NONE, gdr.DT_F32)
    with pytest.raises(TypeError):
        gdr._desc_from(q.half(), g, v)


def test_workspace_size_matches_the_c_call():
    sv, sc = gdr.workspace_size(1, 8192, 16, "scalar", "bf16", "full_save")
    assert sv == 2048 * 123392
    sv2, sc2 = gdr.workspace_size(1, 8192, 16, "none", "bf16", "full_save")
    assert sv2 == sv and sc2 == sc + 2 * 4 * 8192 * 16
    svp, scp = gdr.workspace_size(1, 8192, 16, "vector", "bf16", "recompute", n_seq=3, DK=80, DV=112)
    assert svp == 0 and scp > sc


def test_autograd_operator_refuses_host_tensors():
    q, k, v, g, beta = _args()
    q.requires_grad_(True)
    with pytest.raises(ValueError, match="device tensor"):
        gdr.chunk_gated_delta_rule(q, k, v, g, beta)
