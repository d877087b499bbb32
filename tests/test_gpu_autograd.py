"""The autograd-aware operator (chunk_gated_delta_rule): its gradients are
the library's backward, bit for bit, for whatever adjoints autograd brings
(the output, the final state or both), and they match the oracle's."""
import numpy as np
import pytest

from delta_rule_linear_gdr_amd.inputs import make_inputs, make_packed_inputs
from tests import gdr_testlib as tl

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _leaves(d, names):
    return {n: (None if d[n] is None else d[n].clone().requires_grad_(True)) for n in names}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("gate", ["scalar", "vector", "none"])
@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_autograd_equals_direct_backward_and_oracle(gate, policy):
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    x = make_inputs(1, 200, 2, gate="scalar" if gate == "none" else gate, seed=51,
                    h0_std=0.1, dht_std=0.1)
    if gate == "none":
        x["g"] = np.zeros_like(x["g"])
    d = tl.device_inputs(x)
    if gate == "none":
        d["g"] = None
    lv = _leaves(d, ("q", "k", "v", "g", "beta", "h0"))
    o, ht = gdr.chunk_gated_delta_rule(lv["q"], lv["k"], lv["v"], lv["g"], lv["beta"], lv["h0"],
                                       policy=policy)
    # the loss <o, dO> + <ht, dht> makes autograd hand exactly dO and dht in
    loss = (o.float() * d["dO"].float()).sum() + (ht * d["dht"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    got = {"o": _np(o), "ht": _np(ht)}
    for n, t in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta"),
                 ("dh0", "h0")):
        if lv[t] is not None:
            got[n] = _np(lv[t].grad)
    # the float32 product of a bf16 o with dO casts dO back to bf16 in the
    # adjoint of o, which is dO itself: so the direct call sees the same dO
    _, _, saved = gdr.gdr_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], policy=policy)
    ref = gdr.gdr_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["dO"], d["dht"],
                      saved=saved, policy=policy)
    torch.cuda.synchronize()
    for n, t in ref.items():
        if t is not None:
            assert np.array_equal(got[n], _np(t)), n
    print(f"[autograd] {gate}/{policy}: " + " ".join(
        f"{n}={e:.2e}" for n, e in tl.compare(got, x).items()), flush=True)


def test_autograd_state_only_loss():
    """A loss of the final state alone: the output's adjoint is absent and is
    taken as zero."""
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    x = make_inputs(1, 130, 2, gate="scalar", seed=52, h0_std=0.1, dht_std=0.1)
    x["dO"] = np.zeros_like(x["dO"])
    d = tl.device_inputs(x)
    lv = _leaves(d, ("q", "k", "v", "g", "beta", "h0"))
    _, ht = gdr.chunk_gated_delta_rule(lv["q"], lv["k"], lv["v"], lv["g"], lv["beta"], lv["h0"])
    (ht * d["dht"]).sum().backward()
    torch.cuda.synchronize()
    got = {n: _np(lv[t].grad) for n, t in (("dq", "q"), ("dk", "k"), ("dv", "v"),
                                          ("dg", "g"), ("dbeta", "beta"), ("dh0", "h0"))}
    tl.compare(got, x)
    assert np.all(got["dq"] == 0.0)  # q only reaches the output


def test_autograd_packed():
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    x = make_packed_inputs([70, 0, 150, 64], H=2, gate="vector", seed=53)
    d = tl.device_inputs(x)
    cu = torch.from_numpy(x["cu"]).to("cuda")
    lv = _leaves(d, ("q", "k", "v", "g", "beta", "h0"))
    o, ht = gdr.chunk_gated_delta_rule(lv["q"], lv["k"], lv["v"], lv["g"], lv["beta"], lv["h0"],
                                       cu_seqlens=cu)
    ((o.float() * d["dO"].float()).sum() + (ht * d["dht"]).sum()).backward()
    torch.cuda.synchronize()
    got = {"o": _np(o), "ht": _np(ht)}
    for n, t in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta"),
                 ("dh0", "h0")):
        got[n] = _np(lv[t].grad)
    # tokens past the last sequence: the library leaves them untouched, and
    # autograd's gradient buffers are the library's outputs, so only the
    # covered tokens are compared here
    tail = int(x["cu"][-1])
    assert tail == x["q"].shape[1]
    tl.compare_packed(got, x)


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn2_autograd_equals_direct_backward_and_oracle(policy):
    """chunk_gdn2: autograd's gradients are gdr_bwd_gdn2's bit for bit and
    meet the GDN2 oracle's bar."""
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    from tests.test_gpu_gdn2 import compare_gdn2
    x = make_inputs(1, 200, 2, gate="gdn2", seed=52, gate_mean=3.0, h0_std=0.1, dht_std=0.1)
    d = tl.device_inputs(x)
    d["ers"] = tl.to_dev(x["ers"], torch.bfloat16)
    d["wrt"] = tl.to_dev(x["wrt"], torch.bfloat16)
    lv = _leaves(d, ("q", "k", "v", "g", "ers", "wrt", "h0"))
    o, ht = gdr.chunk_gdn2(lv["q"], lv["k"], lv["v"], lv["g"], lv["ers"], lv["wrt"], lv["h0"],
                           policy=policy)
    loss = (o.float() * d["dO"].float()).sum() + (ht * d["dht"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    got = {"o": _np(o), "ht": _np(ht), "dq": _np(lv["q"].grad), "dk": _np(lv["k"].grad),
           "dv": _np(lv["v"].grad), "dg": _np(lv["g"].grad), "ders": _np(lv["ers"].grad),
           "dwrt": _np(lv["wrt"].grad), "dh0": _np(lv["h0"].grad)}
    _, _, saved = gdr.gdr_fwd_gdn2(d["q"], d["k"], d["v"], d["g"], d["ers"], d["wrt"], d["h0"],
                                   policy=policy)
    ref = gdr.gdr_bwd_gdn2(d["q"], d["k"], d["v"], d["g"], d["ers"], d["wrt"], d["h0"], d["dO"],
                           d["dht"], saved=saved, policy=policy)
    torch.cuda.synchronize()
    for n, r in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dg", "dg"), ("ders", "derase"),
                 ("dwrt", "dwrite"), ("dh0", "dh0")):
        assert np.array_equal(got[n], _np(ref[r])), n
    compare_gdn2(got, x)


def test_gdn2_autograd_packed():
    """chunk_gdn2 over a packed batch that covers every token (autograd's
    gradient buffers are the library's outputs): per-sequence states, and the
    GDN2 oracle's bar per sequence."""
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    from tests.test_gpu_gdn2 import compare_gdn2_packed
    x = make_packed_inputs([90, 0, 150], H=2, gate="gdn2", seed=53, gate_mean=3.0)
    d = tl.device_inputs(x)
    d["ers"] = tl.to_dev(x["ers"], torch.bfloat16)
    d["wrt"] = tl.to_dev(x["wrt"], torch.bfloat16)
    cu = torch.from_numpy(x["cu"]).to("cuda")
    lv = _leaves(d, ("q", "k", "v", "g", "ers", "wrt", "h0"))
    o, ht = gdr.chunk_gdn2(lv["q"], lv["k"], lv["v"], lv["g"], lv["ers"], lv["wrt"], lv["h0"],
                           cu_seqlens=cu)
    loss = (o.float() * d["dO"].float()).sum() + (ht * d["dht"]).sum()
    loss.backward()
    torch.cuda.synchronize()
    got = {"o": _np(o), "ht": _np(ht), "dq": _np(lv["q"].grad), "dk": _np(lv["k"].grad),
           "dv": _np(lv["v"].grad), "dg": _np(lv["g"].grad), "ders": _np(lv["ers"].grad),
           "dwrt": _np(lv["wrt"].grad), "dh0": _np(lv["h0"].grad)}
    compare_gdn2_packed(got, x)
