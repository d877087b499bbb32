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
    with pytest.raises(TypeError, match="k dtype"):
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
    assert sv == 2048 * 115200
    sv2, sc2 = gdr.workspace_size(1, 8192, 16, "none", "bf16", "full_save")
    assert sv2 == sv and sc2 == sc + 2 * 4 * 8192 * 16
    svp, scp = gdr.workspace_size(1, 8192, 16, "vector", "bf16", "recompute", n_seq=3, DK=80, DV=112)
    assert svp == 0 and scp > sc


def test_autograd_operator_refuses_host_tensors():
    q, k, v, g, beta = _args()
    q.requires_grad_(True)
    with pytest.raises(ValueError, match="device tensor"):
        gdr.chunk_gated_delta_rule(q, k, v, g, beta)


def _on_device(monkeypatch):
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))


def _bwd_args(B=1, T=64, H=2, dk=128, dv=128, vec=False):
    q, k, v, g, beta = _args(B, T, H, dk, dv, vec)
    dO = _t(B, T, H, dv)
    return q, k, v, g, beta, dO


@pytest.mark.parametrize("case, err, match", [
    ("k_narrower", ValueError, "k shape"),
    ("g_trailing_1", ValueError, "g shape"),
    ("beta_short", ValueError, "beta shape"),
    ("h0_bf16", TypeError, "h0 dtype"),
    ("h0_wrong_heads", ValueError, "h0 shape"),
    ("v_wrong_tokens", ValueError, "v shape"),
])
def test_forward_shapes_and_dtypes_are_checked(monkeypatch, case, err, match):
    """Every tensor is checked against (B, T, H, DK, DV) before a launch: a
    mismatch would otherwise let the kernels read past a tensor."""
    _on_device(monkeypatch)
    q, k, v, g, beta = _args()
    h0 = None
    if case == "k_narrower":
        k = _t(1, 64, 2, 96)
    elif case == "g_trailing_1":
        g = _t(1, 64, 2, 1, dtype=torch.float32)
    elif case == "beta_short":
        beta = _t(1, 63, 2)
    elif case == "h0_bf16":
        h0 = _t(1, 2, 128, 128)
    elif case == "h0_wrong_heads":
        h0 = _t(1, 3, 128, 128, dtype=torch.float32)
    elif case == "v_wrong_tokens":
        v = _t(1, 65, 2, 128)
    with pytest.raises(err, match=match):
        gdr.gdr_fwd(q, k, v, g, beta, h0)


@pytest.mark.parametrize("case, err, match", [
    ("dht_bf16", TypeError, "dht dtype"),
    ("dO_wide", ValueError, "dO shape"),
    ("dO_dtype", TypeError, "dO dtype"),
    ("out_dq_shape", ValueError, "dq shape"),
    ("out_dg_dtype", TypeError, "dg dtype"),
    ("out_dh0_shape", ValueError, "dh0 shape"),
    ("out_missing_dg", ValueError, "dg"),
    ("scratch_float", TypeError, "scratch dtype"),
    ("saved_small", ValueError, "saved holds"),
    ("saved_missing", ValueError, "full-save"),
])
def test_backward_shapes_and_dtypes_are_checked(monkeypatch, case, err, match):
    _on_device(monkeypatch)
    q, k, v, g, beta, dO = _bwd_args()
    dht, out, scratch, saved, policy = None, None, None, None, "recompute"
    full = dict(dq=_t(1, 64, 2, 128), dk=_t(1, 64, 2, 128), dv=_t(1, 64, 2, 128),
                dg=_t(1, 64, 2, dtype=torch.float32), dbeta=_t(1, 64, 2),
                dh0=_t(1, 2, 128, 128, dtype=torch.float32))
    if case == "dht_bf16":
        dht = _t(1, 2, 128, 128)
    elif case == "dO_wide":
        dO = _t(1, 64, 2, 129)
    elif case == "dO_dtype":
        dO = dO.float()
    elif case == "out_dq_shape":
        out = dict(full, dq=_t(1, 64, 2, 64))
    elif case == "out_dg_dtype":
        out = dict(full, dg=_t(1, 64, 2))
    elif case == "out_dh0_shape":
        out = dict(full, dh0=_t(2, 2, 128, 128, dtype=torch.float32))
    elif case == "out_missing_dg":
        out = dict(full, dg=None)
    elif case == "scratch_float":
        scratch = torch.zeros(1 << 20, dtype=torch.float32)
    elif case == "saved_small":
        policy, saved = "full_save", torch.zeros(1024, dtype=torch.uint8)
    elif case == "saved_missing":
        policy = "full_save"
    with pytest.raises(err, match=match):
        gdr.gdr_bwd(q, k, v, g, beta, None, dO, dht, saved=saved, policy=policy,
                    scratch=scratch, out=out)


def test_packed_states_follow_the_sequence_count(monkeypatch):
    _on_device(monkeypatch)
    q, k, v, g, beta = _args(T=128)
    cu = torch.tensor([0, 50, 128], dtype=torch.int64)
    with pytest.raises(ValueError, match="h0 shape"):
        gdr.gdr_fwd(q, k, v, g, beta, _t(1, 2, 128, 128, dtype=torch.float32), cu_seqlens=cu)
