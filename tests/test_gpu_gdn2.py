"""GPU parity of GDN2 (per-key-channel decay with independent erase and
write gates) through the C ABI against the fp64 GDN2 oracle on identical
seeded inputs. Bar (paper Sec. 4.5): 0.8% relative L2 for outputs, states
and ordinary gradients, 2% for the gate and erase/write gradients."""
import numpy as np
import pytest

import oracle
from delta_rule_linear_gdr_amd.inputs import make_inputs
from tests import gdr_testlib as tl

pytestmark = pytest.mark.gpu

TOL = dict(tl.TOL, ders=0.02, dwrt=0.02)


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run_gdn2(x, policy="recompute", use_states=True):
    import torch
    import delta_rule_linear_gdr_amd as gdr
    d = tl.device_inputs(x)
    e = tl.to_dev(x["ers"], torch.bfloat16)
    w = tl.to_dev(x["wrt"], torch.bfloat16)
    h0 = d["h0"] if use_states else None
    dht = d["dht"] if use_states else None
    o, ht, saved = gdr.gdr_fwd_gdn2(d["q"], d["k"], d["v"], d["g"], e, w, h0, policy=policy)
    gr = gdr.gdr_bwd_gdn2(d["q"], d["k"], d["v"], d["g"], e, w, h0, d["dO"], dht, saved=saved,
                          policy=policy)
    torch.cuda.synchronize()
    out = {"o": o, "ht": ht, "dq": gr["dq"], "dk": gr["dk"], "dv": gr["dv"], "dg": gr["dg"],
           "ders": gr["derase"], "dwrt": gr["dwrite"], "dh0": gr["dh0"]}
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items() if t is not None}


def compare_gdn2(gpu, x, use_states=True, per_head=False):
    h0 = x["h0"] if use_states else None
    dht = x["dht"] if use_states else None
    o, ht = oracle.gdn2_fwd(x["q"], x["k"], x["v"], x["g"], x["ers"], x["wrt"], h0)
    ref = oracle.gdn2_bwd(x["q"], x["k"], x["v"], x["g"], x["ers"], x["wrt"], h0, x["dO"], dht)
    ref.update(o=o, ht=ht)
    errs = {}
    B, _, H = x["q"].shape[:3]
    for n in ("o", "ht", "dq", "dk", "dv", "dg", "ders", "dwrt", "dh0"):
        if n not in gpu:
            continue
        errs[n] = tl.check(n, gpu[n], ref[n], tol=TOL[n])
        if per_head:
            for b in range(B):
                for h in range(H):
                    sl = (b, h) if n in ("ht", "dh0") else (b, slice(None), h)
                    tl.check(n, gpu[n][sl], ref[n][sl], tol=TOL[n])
    return errs


def _report(tag, errs):
    print(f"[gdn2] {tag}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn2_small_with_states(policy):
    _need_gpu()
    x = make_inputs(1, 256, 2, gate="gdn2", dtype="bf16", seed=31, gate_mean=3.0,
                    h0_std=0.1, dht_std=0.1)
    _report(f"1x256x2/{policy}", compare_gdn2(run_gdn2(x, policy), x))


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn2_ragged_two_sequences(policy):
    """T = 300: a ragged last chunk right before the second batch entry."""
    _need_gpu()
    x = make_inputs(2, 300, 3, gate="gdn2", dtype="bf16", seed=32, gate_mean=3.0,
                    h0_std=0.1, dht_std=0.1)
    _report(f"2x300x3/{policy}", compare_gdn2(run_gdn2(x, policy), x, per_head=True))


def test_gdn2_2048x16_all_heads():
    _need_gpu()
    x = make_inputs(1, 2048, 16, gate="gdn2", dtype="bf16", seed=0, gate_mean=3.0)
    _report("1x2048x16/recompute", compare_gdn2(run_gdn2(x), x, per_head=True))


def test_gdn2_8192x16_all_heads():
    """The pages' headline shape, every head."""
    _need_gpu()
    x = make_inputs(1, 8192, 16, gate="gdn2", dtype="bf16", seed=0, gate_mean=3.0, h0_std=0.1)
    _report("1x8192x16/recompute", compare_gdn2(run_gdn2(x), x, per_head=True))


def test_gdn2_strong_decay_and_zero_gates():
    """Per-token decays around e^-4 (16-token windows, boundary pivots), with
    erase gates switched off on some (token, key) entries and write gates on
    some (token, value) entries."""
    _need_gpu()
    x = make_inputs(1, 256, 2, gate="gdn2", dtype="bf16", seed=33, gate_mean=-4.0,
                    h0_std=0.1, dht_std=0.1)
    x["ers"] = x["ers"].copy()
    x["wrt"] = x["wrt"].copy()
    x["ers"][:, ::3, :, ::2] = 0.0
    x["wrt"][:, 1::5, :, 1::3] = 0.0
    for pol in ("recompute", "full_save"):
        _report(f"strong/{pol}", compare_gdn2(run_gdn2(x, pol), x))


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn2_with_shared_gates_equals_the_vector_gate_path(policy):
    """erase = write = beta in every channel: GDN2 is the vector-gate
    (KDA) recurrence, and the kernels do the same arithmetic on the same
    values, so o, ht, dq, dk, dv, dg, dh0 equal the KDA call's bit for bit;
    the channel sums of derase and dwrite match its dbeta to the bar."""
    _need_gpu()
    x = make_inputs(1, 200, 3, gate="vector", dtype="bf16", seed=34, gate_mean=3.0,
                    h0_std=0.1, dht_std=0.1)
    x["ers"] = np.repeat(x["beta"][..., None], 128, axis=-1)
    x["wrt"] = np.repeat(x["beta"][..., None], 128, axis=-1)
    kda = tl.run_gpu(x, policy)
    g2 = run_gdn2(x, policy)
    for n in ("o", "ht", "dq", "dk", "dv", "dg", "dh0"):
        assert np.array_equal(g2[n], kda[n]), n
    tl.check("dbeta", g2["ders"].sum(-1) + g2["dwrt"].sum(-1), kda["dbeta"])


def test_gdn2_without_states():
    _need_gpu()
    x = make_inputs(1, 192, 2, gate="gdn2", dtype="bf16", seed=35, gate_mean=3.0)
    _report("no states", compare_gdn2(run_gdn2(x, use_states=False), x, use_states=False))
