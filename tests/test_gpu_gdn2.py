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


def test_gdn2_repeatable_bits():
    """Two identical calls give identical bits (the GDN2 local kernel reads
    its D^T and Hb^T operands transposed from shared tiles in LDS)."""
    _need_gpu()
    x = make_inputs(2, 300, 3, gate="gdn2", dtype="bf16", seed=33, gate_mean=3.0,
                    h0_std=0.1, dht_std=0.1)
    a, b = run_gdn2(x), run_gdn2(x)
    for n in a:
        if a[n] is not None:
            np.testing.assert_array_equal(a[n], b[n], err_msg=f"repeat {n}")


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


# ------------------------------------- packed batches and other widths (GDN2)

def run_gdn2_packed(x, policy="recompute"):
    """Packed GDN2 forward + backward; o and the gradient outputs prefilled
    with a sentinel that tokens outside every sequence must keep."""
    import torch
    import delta_rule_linear_gdr_amd as gdr
    d = tl.device_inputs(x)
    e = tl.to_dev(x["ers"], torch.bfloat16)
    w = tl.to_dev(x["wrt"], torch.bfloat16)
    cu = torch.from_numpy(x["cu"]).to("cuda")
    o, ht, saved = gdr.gdr_fwd_gdn2(d["q"], d["k"], d["v"], d["g"], e, w, d["h0"], policy=policy,
                                    cu_seqlens=cu, o=torch.full_like(d["v"], tl.SENTINEL))
    out = {n: torch.full_like(t, tl.SENTINEL) for n, t in
           (("dq", d["q"]), ("dk", d["k"]), ("dv", d["v"]), ("dg", d["g"]), ("derase", e),
            ("dwrite", w))}
    out["dh0"] = torch.empty_like(d["h0"])
    gr = gdr.gdr_bwd_gdn2(d["q"], d["k"], d["v"], d["g"], e, w, d["h0"], d["dO"], d["dht"],
                          saved=saved, policy=policy, out=out, cu_seqlens=cu)
    torch.cuda.synchronize()
    res = {"o": o, "ht": ht, "dq": gr["dq"], "dk": gr["dk"], "dv": gr["dv"], "dg": gr["dg"],
           "ders": gr["derase"], "dwrt": gr["dwrite"], "dh0": gr["dh0"]}
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in res.items()}


def compare_gdn2_packed(gpu, x):
    """Each sequence is its own GDN2 problem with its own h0 and dht (an empty
    one passes its state through); acceptance per tensor over the covered
    tokens, and the sentinel kept past the last sequence."""
    cu = x["cu"]
    H = x["q"].shape[2]
    got, ref = {}, {}
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        for h in range(H):
            sl = lambda t: t[:, a:b, h:h + 1]       # noqa: E731
            st = lambda t: t[i:i + 1, h:h + 1]      # noqa: E731
            if a == b:
                r = {"ht": st(x["h0"]), "dh0": st(x["dht"])}
            else:
                o, ht = oracle.gdn2_fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["ers"]),
                                        sl(x["wrt"]), st(x["h0"]))
                r = oracle.gdn2_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["ers"]),
                                    sl(x["wrt"]), st(x["h0"]), sl(x["dO"]), st(x["dht"]))
                r.update(o=o, ht=ht)
            for n, arr in r.items():
                gg = gpu[n][i:i + 1, h:h + 1] if n in ("ht", "dh0") else gpu[n][:, a:b, h:h + 1]
                got.setdefault(n, []).append(gg.ravel())
                ref.setdefault(n, []).append(np.asarray(arr).ravel())
    errs = {n: tl.check(n, np.concatenate(got[n]), np.concatenate(ref[n]), tol=TOL[n]) for n in got}
    tail = int(cu[-1])
    for n in ("o", "dq", "dk", "dv", "dg", "ders", "dwrt"):
        assert np.all(gpu[n][:, tail:] == tl.SENTINEL), f"{n}: tokens past the last sequence written"
    return errs


def _narrow(x, dk, dv, states=True):
    """Cut seeded 128-wide inputs to dk keys and dv values (the shortened keys
    are not renormalised: the recurrence takes any key)."""
    for n in ("q", "k", "g", "ers"):
        x[n] = np.ascontiguousarray(x[n][..., :dk])
    for n in ("v", "dO", "wrt"):
        x[n] = np.ascontiguousarray(x[n][..., :dv])
    if states:
        for n in ("h0", "dht"):
            x[n] = np.ascontiguousarray(x[n][:, :, :dk, :dv])
    return x


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn2_packed_mixed_lengths(policy):
    """Sequences of 100, 0, 129 and 64 tokens (ragged chunks, an empty
    sequence, chunks that start mid-chunk) in a row of 320 tokens whose last
    27 belong to no sequence."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    x = make_packed_inputs([100, 0, 129, 64], H=2, gate="gdn2", seed=36, gate_mean=3.0, cover=320)
    _report(f"packed/{policy}", compare_gdn2_packed(run_gdn2_packed(x, policy), x))


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn2_packed_narrow_widths(policy):
    """A packed batch at key width 80 and value width 112."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    x = _narrow(make_packed_inputs([70, 0, 130], H=2, gate="gdn2", seed=37, gate_mean=3.0), 80, 112)
    _report(f"packed/80x112/{policy}", compare_gdn2_packed(run_gdn2_packed(x, policy), x))


def test_gdn2_packed_value_blocks():
    """A packed batch at key width 64 and value width 160 (a 128-wide value
    block and a 32-wide one, each zero-padded), with a tail of tokens outside
    every sequence: padding, value blocks and the sequence table together."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs, round_bf16, round_fp32
    x = make_packed_inputs([50, 0, 90], H=2, gate="gdn2", seed=38, gate_mean=3.0, cover=160)
    # values and value-side tensors widened to 160 with fresh draws (any value is valid)
    rng = np.random.default_rng(39)
    wide = lambda a, extra: np.ascontiguousarray(np.concatenate([a, extra], axis=-1))  # noqa: E731
    T, H = x["q"].shape[1:3]
    x["v"] = wide(x["v"], round_bf16(rng.standard_normal((1, T, H, 32))))
    x["dO"] = wide(x["dO"], round_bf16(rng.standard_normal((1, T, H, 32))))
    x["wrt"] = wide(x["wrt"], round_bf16(1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, H, 32))))))
    n = len(x["cu"]) - 1
    x["h0"] = wide(x["h0"], round_fp32(0.1 * rng.standard_normal((n, H, 128, 32))))
    x["dht"] = wide(x["dht"], round_fp32(0.1 * rng.standard_normal((n, H, 128, 32))))
    x = _narrow(x, 64, 160)
    for pol in ("recompute", "full_save"):
        _report(f"packed/64x160/{pol}", compare_gdn2_packed(run_gdn2_packed(x, pol), x))


@pytest.mark.parametrize("dk,dv", [(80, 112), (96, 80), (128, 160), (64, 300)])
def test_gdn2_other_widths(dk, dv):
    """Key widths below 128 through zero-padded copies; value widths above
    128 as 128-wide value blocks (the erase gate's gradient, a key-side
    gradient, summed over the blocks; the write gate's taken per block)."""
    _need_gpu()
    x = make_inputs(2, 100, 2, DK=dk, DV=dv, gate="gdn2", dtype="bf16", seed=38, gate_mean=3.0,
                    h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"{dk}x{dv}/{pol}", compare_gdn2(run_gdn2(x, pol), x, per_head=True))
