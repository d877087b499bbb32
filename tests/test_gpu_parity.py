"""GPU parity: the HIP path through the C ABI against the fp64 token oracle on
identical seeded inputs, at the five workloads and on the edge cases."""
import numpy as np
import pytest

from delta_rule_linear_gdr_amd.inputs import WORKLOADS, make_inputs
from tests import gdr_testlib as tl

pytestmark = pytest.mark.gpu


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(tag, errs):
    print(f"[parity] {tag}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn_512x4_fp32(policy):
    _need_gpu()
    x = WORKLOADS["gdn_1x512x4_fp32"].make()
    gpu = tl.run_gpu(x, policy)
    _report(f"gdn_1x512x4_fp32/{policy}", tl.compare(gpu, x))


def test_gdn_2048x16_full_save():
    _need_gpu()
    x = WORKLOADS["gdn_1x2048x16"].make()
    gpu = tl.run_gpu(x, "full_save")
    _report("gdn_1x2048x16/full_save", tl.compare(gpu, x))


@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_gdn_8192x16_all_heads(policy):
    _need_gpu()
    x = WORKLOADS["gdn_1x8192x16"].make()
    gpu = tl.run_gpu(x, policy)
    _report(f"gdn_1x8192x16/{policy}", tl.compare_all_heads(gpu, x))


def test_kda_2x2048x16_all_heads():
    _need_gpu()
    x = WORKLOADS["kda_2x2048x16"].make()
    gpu = tl.run_gpu(x, "recompute")
    _report("kda_2x2048x16/recompute", tl.compare_all_heads(gpu, x))


def test_kda_8192x16_h0_all_heads():
    _need_gpu()
    x = WORKLOADS["kda_1x8192x16"].make()
    gpu = tl.run_gpu(x, "recompute")
    _report("kda_1x8192x16/recompute", tl.compare_all_heads(gpu, x))


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_four_head_shapes(gate):
    """The two four-head shapes of the pages' six-shape evaluation that the
    workloads above do not cover, both policies; (1,8192,4) on sampled heads."""
    _need_gpu()
    mean = 4.0 if gate == "scalar" else 3.0
    x = make_inputs(1, 2048, 4, gate=gate, dtype="bf16", seed=0, gate_mean=mean)
    for pol in ("recompute", "full_save"):
        _report(f"{gate}_1x2048x4/{pol}", tl.compare(tl.run_gpu(x, pol), x))
    x = make_inputs(1, 8192, 4, gate=gate, dtype="bf16", seed=0, gate_mean=mean)
    for pol in ("recompute", "full_save"):
        _report(f"{gate}_1x8192x4/{pol}", tl.compare(tl.run_gpu(x, pol), x, heads=[(0, 1), (0, 3)]))


# ------------------------------------------------------------------ edges

def _edge(gate, T=256, H=2, B=1, seed=3, **kw):
    x = make_inputs(B, T, H, gate=gate, dtype="bf16", seed=seed,
                    gate_mean=4.0 if gate == "scalar" else 3.0, **kw)
    return x


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_single_chunk(gate):
    _need_gpu()
    x = _edge(gate, T=64, H=3)
    _report(f"single_chunk/{gate}", tl.compare(tl.run_gpu(x), x))


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_nonzero_initial_and_terminal_state(gate):
    _need_gpu()
    x = _edge(gate, h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"h0_dht/{gate}/{pol}", tl.compare(tl.run_gpu(x, pol), x))


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_zero_and_tiny_beta(gate):
    _need_gpu()
    x = _edge(gate, h0_std=0.1, dht_std=0.1)
    x["beta"] = x["beta"].copy()
    x["beta"][:, ::3] = 0.0
    x["beta"][:, 1::7] = 1e-8 if x["dtype"] == "fp32" else np.float64(np.float32(1e-8))
    from delta_rule_linear_gdr_amd.inputs import round_to
    x["beta"] = round_to(x["beta"], x["dtype"])
    _report(f"zero_tiny_beta/{gate}", tl.compare(tl.run_gpu(x), x))


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_all_zero_beta(gate):
    _need_gpu()
    x = _edge(gate, h0_std=0.1, dht_std=0.1)
    x["beta"] = np.zeros_like(x["beta"])
    _report(f"beta0/{gate}", tl.compare(tl.run_gpu(x), x))


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_strong_decay(gate):
    _need_gpu()
    x = make_inputs(1, 256, 2, gate=gate, dtype="bf16", seed=5, gate_mean=0.0)
    _report(f"strong_decay/{gate}", tl.compare(tl.run_gpu(x), x))


def test_deterministic_and_policy_independent():
    _need_gpu()
    x = _edge("vector", T=512, H=4, h0_std=0.1, dht_std=0.1)
    a = tl.run_gpu(x, "recompute")
    b = tl.run_gpu(x, "recompute")
    c = tl.run_gpu(x, "full_save")
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=f"repeat {n}")
        np.testing.assert_array_equal(a[n], c[n], err_msg=f"policy {n}")


@pytest.mark.parametrize("gate", ["scalar", "vector", "none"])
@pytest.mark.parametrize("wy7", [False, True])
def test_repeatable_bits(gate, wy7):
    """Two identical calls give identical bits, for every local kernel (the
    persistent scalar-gate one, the per-chunk vector-gate one, DeltaNet, and
    the seven-product producers), with a ragged last chunk. The local kernels
    exchange their operand tiles through LDS, some read transposed; a tile
    read before its writer finished would show here as a difference."""
    _need_gpu()
    x = _edge("scalar" if gate == "none" else gate, T=300, H=3, h0_std=0.1, dht_std=0.1)
    nogate = gate == "none"
    if nogate:
        x["g"] = np.zeros_like(x["g"])
    a = tl.run_gpu(x, "recompute", wy7=wy7, nogate=nogate)
    b = tl.run_gpu(x, "recompute", wy7=wy7, nogate=nogate)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=f"repeat {n}")


@pytest.mark.parametrize("gate,wy7", [("vector", False), ("scalar", True)])
def test_repeatable_bits_staggered_launch(gate, wy7):
    """At (1,8192,16) the per-chunk local launches run 2,048 workgroups, eight
    rounds of one per CU, so half the CUs start their first workgroup late.
    The delay changes only timing: two calls still give identical bits."""
    _need_gpu()
    x = _edge(gate, T=8192, H=16, h0_std=0.1, dht_std=0.1)
    a = tl.run_gpu(x, "recompute", wy7=wy7)
    b = tl.run_gpu(x, "recompute", wy7=wy7)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=f"repeat {n}")


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_wy7_policy_independent(gate):
    """The seven-product backward under full save forms A from the saved A^T
    (an exact transpose); under recompute prep writes A itself. Both give
    the same bits, including a ragged last chunk."""
    _need_gpu()
    x = _edge(gate, T=300, H=3, h0_std=0.1, dht_std=0.1)
    a = tl.run_gpu(x, "recompute", wy7=True)
    c = tl.run_gpu(x, "full_save", wy7=True)
    for n in a:
        np.testing.assert_array_equal(a[n], c[n], err_msg=f"policy {n}")
    _report(f"wy7 policies/{gate}", tl.compare(c, x))


def test_unsupported_width_raises():
    """A key width above 128 is refused before anything is launched."""
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    x = _edge("scalar", T=128)
    d = tl.device_inputs(x)
    wide = lambda t: torch.cat([t, t[..., :64]], dim=-1).contiguous()  # noqa: E731
    with pytest.raises(gdr.GdrError) as ei:
        gdr.gdr_fwd(wide(d["q"]), wide(d["k"]), d["v"], d["g"], d["beta"])
    assert ei.value.status == -2


# ---------------------------------------------- ragged last chunk (T % 64 != 0)

@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_ragged_tail(gate):
    """Lengths that end inside a chunk, two batch entries (the ragged chunk of
    entry 0 sits right before entry 1's tokens), both policies, nonzero h0 and
    dht: the missing rows must neither be read nor written."""
    _need_gpu()
    for T in (1, 63, 65, 100, 191, 257):
        x = _edge(gate, T=T, H=2, B=2, seed=11, h0_std=0.1, dht_std=0.1)
        for pol in ("recompute", "full_save"):
            _report(f"ragged/{gate}/T={T}/{pol}", tl.compare(tl.run_gpu(x, pol), x))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ragged_chunk_late_in_a_persistent_walk(dtype):
    """(1, 8292, 2): 130 chunks x 2 heads = 260 (chunk, head) items, more
    than one per workgroup of a one-per-CU launch, unevenly: head 1's ragged
    last chunk (100 rows) is a later item of its workgroup, after a prefetch
    and with the previous item's deferred reductions pending. Head 1 is
    compared in full."""
    _need_gpu()
    x = make_inputs(1, 8292, 2, gate="scalar", dtype=dtype, seed=13, h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"persistent-ragged/{dtype}/{pol}", tl.compare(tl.run_gpu(x, pol), x, heads=[(0, 1)]))


def test_ragged_tail_fp32():
    _need_gpu()
    x = make_inputs(2, 100, 3, gate="scalar", dtype="fp32", seed=12, gate_mean=4.0, h0_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"ragged/fp32/T=100/{pol}", tl.compare(tl.run_gpu(x, pol), x))


# ------------------------------------------------- seven-product ablation

@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_wy7_gdn_8192x16_sampled_heads(policy):
    """The expanded seven-product producer gives the same gradients."""
    _need_gpu()
    x = WORKLOADS["gdn_1x8192x16"].make()
    gpu = tl.run_gpu(x, policy, wy7=True)
    _report(f"wy7 gdn_1x8192x16/{policy}", tl.compare(gpu, x, heads=[(0, 0), (0, 9)]))


def test_wy7_kda_2x2048x16():
    _need_gpu()
    x = WORKLOADS["kda_2x2048x16"].make()
    gpu = tl.run_gpu(x, "recompute", wy7=True)
    _report("wy7 kda_2x2048x16/recompute", tl.compare(gpu, x, heads=[(0, 3), (1, 12)]))


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_wy7_edges_fp32_and_strong_decay(gate):
    _need_gpu()
    x = make_inputs(1, 256, 2, gate=gate, dtype="fp32", seed=7,
                    gate_mean=0.0, h0_std=0.1, dht_std=0.1)
    _report(f"wy7 strong_decay_fp32/{gate}", tl.compare(tl.run_gpu(x, wy7=True), x))


# ------------------------------------------------ packed variable-length batches

@pytest.mark.gpu
@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_packed_mixed_lengths(gate):
    """Sequences of mixed lengths in one row (empty ones, one token, ragged
    and whole chunks, sequences starting inside a chunk), each with its own
    h0 and dht, a tail of tokens belonging to no sequence; both policies."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    lengths = [100, 0, 64, 1, 191, 0, 257, 63]
    x = make_packed_inputs(lengths, H=2, gate=gate, seed=21,
                           gate_mean=4.0 if gate == "scalar" else 3.0, cover=sum(lengths) + 37)
    for pol in ("recompute", "full_save"):
        _report(f"packed/{gate}/{pol}", tl.compare_packed(tl.run_gpu_packed(x, pol), x))


@pytest.mark.gpu
def test_packed_many_short_sequences():
    """Forty sequences of random lengths (uniform cut points, some empty) over
    2000 tokens: many chunk slots, most sequences ragged."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs, packed_lengths
    x = make_packed_inputs(packed_lengths(2000, 40, seed=5), H=2, gate="scalar", seed=22)
    _report("packed/many", tl.compare_packed(tl.run_gpu_packed(x), x))


@pytest.mark.gpu
@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_packed_8192x16_sampled_heads(gate):
    """Full length and width (8192 tokens, 16 heads) split into sequences of
    mixed lengths; the oracle checks two heads of every sequence."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    lengths = [1000, 3000, 37, 4155]
    x = make_packed_inputs(lengths, H=16, gate=gate, seed=23,
                           gate_mean=4.0 if gate == "scalar" else 3.0)
    _report(f"packed8192/{gate}", tl.compare_packed(tl.run_gpu_packed(x), x, heads=(0, 15)))


@pytest.mark.gpu
def test_packed_single_sequence_matches_regular_batch():
    """One sequence covering the row is the regular problem: identical
    results, bit for bit (same kernels, same tiles, same order)."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    x = make_packed_inputs([300], H=2, gate="vector", seed=24, gate_mean=3.0)
    for pol in ("recompute", "full_save"):
        p = tl.run_gpu_packed(x, pol)
        r = tl.run_gpu(x, pol)
        for n in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
            assert np.array_equal(p[n], r[n]), n


# ---------------------------------------- strong decay under the vector gate

@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_kda_strong_decay_windowed(dtype):
    """Per-key log decays around -4 per token (log-sigmoid of N(-4, 1)): a
    64-token chunk spans a range near 256, far past what chunk-wide centred
    factors can hold in fp32, a 16-token window about 60. Both policies,
    the seven-product producer, nonzero states and a ragged last chunk."""
    _need_gpu()
    x = make_inputs(1, 300, 2, gate="vector", dtype=dtype, seed=31, gate_mean=-4.0,
                    h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"kda_strong/{dtype}/{pol}", tl.compare(tl.run_gpu(x, pol), x))
    _report(f"kda_strong/{dtype}/wy7", tl.compare(tl.run_gpu(x, wy7=True), x))


@pytest.mark.gpu
@pytest.mark.parametrize("decay", [-5.0, -8.0, -10.0])
def test_kda_decay_up_to_the_window_limit(decay):
    """Every log decay the same, up to -10 (a 16-token window spans 150, its
    factors reach exp(75)): the edge of the vector gate's contract. At -5 and
    -8 a 32-token window would span 155 and 248: past fp32 for the latter.
    Both policies and the seven-product producer."""
    _need_gpu()
    x = make_inputs(1, 256, 2, gate="vector", dtype="bf16", seed=32, h0_std=0.1, dht_std=0.1)
    x["g"] = np.full_like(x["g"], decay)
    for pol in ("recompute", "full_save"):
        _report(f"kda_limit/{decay}/{pol}", tl.compare(tl.run_gpu(x, pol), x))
    _report(f"kda_limit/{decay}/wy7", tl.compare(tl.run_gpu(x, wy7=True), x))


@pytest.mark.gpu
def test_kda_8192x16_strong_decay_sampled_heads():
    """Full length and width with log decays around -3 per token."""
    _need_gpu()
    x = make_inputs(1, 8192, 16, gate="vector", dtype="bf16", seed=33, gate_mean=-3.0,
                    h0_std=0.1)
    gpu = tl.run_gpu(x)
    _report("kda_8192x16_strong", tl.compare(gpu, x, heads=[(0, 0), (0, 9)]))


# --------------------------------------------------- DeltaNet (no decay)

@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_deltanet_no_gate(dtype):
    """g = None runs the recurrence without decay (the oracle with g = 0): a
    ragged last chunk, nonzero states, both policies and the seven-product
    producer; dg is not produced. Equal, bit for bit, to the scalar-gate call
    with an all-zero g."""
    _need_gpu()
    x = make_inputs(1, 300, 2, gate="scalar", dtype=dtype, seed=41, h0_std=0.1, dht_std=0.1)
    x["g"] = np.zeros_like(x["g"])
    for pol in ("recompute", "full_save"):
        got = tl.run_gpu(x, pol, nogate=True)
        assert "dg" not in got
        _report(f"deltanet/{dtype}/{pol}", tl.compare(got, x))
        ref = tl.run_gpu(x, pol)
        for n in got:
            assert np.array_equal(got[n], ref[n]), n
    _report(f"deltanet/{dtype}/wy7", tl.compare(tl.run_gpu(x, wy7=True, nogate=True), x))


@pytest.mark.gpu
def test_deltanet_packed():
    """DeltaNet over a packed batch (per-sequence states)."""
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    x = make_packed_inputs([100, 0, 129, 64], H=2, gate="scalar", seed=42)
    x["g"] = np.zeros_like(x["g"])
    d = tl.device_inputs(x)
    cu = torch.from_numpy(x["cu"]).to("cuda")
    o, ht, saved = gdr.gdr_fwd(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], cu_seqlens=cu)
    gr = gdr.gdr_bwd(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], d["dO"], d["dht"],
                     cu_seqlens=cu)
    torch.cuda.synchronize()
    got = {n: t.float().cpu().numpy().astype(np.float64)
           for n, t in {"o": o, "ht": ht, **gr}.items() if t is not None}
    ref = tl.oracle_packed(x)
    for n in ("o", "ht", "dq", "dk", "dv", "dbeta", "dh0"):
        g_all, r_all = [], []
        for (i, h), r in ref.items():
            if n not in r:
                continue
            a, b = int(x["cu"][i]), int(x["cu"][i + 1])
            g_all.append((got[n][i:i + 1, h:h + 1] if n in ("ht", "dh0") else got[n][:, a:b, h:h + 1]).ravel())
            r_all.append(np.asarray(r[n]).ravel())
        tl.check(n, np.concatenate(g_all), np.concatenate(r_all))


# ---------------------------------------------- key / value widths below 128

@pytest.mark.gpu
@pytest.mark.parametrize("gate", ["scalar", "vector"])
@pytest.mark.parametrize("dk,dv", [(80, 112), (96, 80)])
def test_narrow_widths(gate, dk, dv):
    """The pages' extended-test widths (80/112, 96/80) through zero-padded
    copies: two batch entries, a ragged last chunk, nonzero states, both
    policies."""
    _need_gpu()
    x = make_inputs(2, 100, 2, DK=dk, DV=dv, gate=gate, dtype="bf16", seed=51,
                    gate_mean=4.0 if gate == "scalar" else 3.0, h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"narrow/{gate}/{dk}x{dv}/{pol}", tl.compare(tl.run_gpu(x, pol), x))


@pytest.mark.gpu
def test_narrow_widths_fp32_wy7_and_packed():
    """fp32 storage and the seven-product producer at 64/96, and a packed
    batch at 80/112 with a tail of tokens outside every sequence."""
    _need_gpu()
    x = make_inputs(1, 150, 2, DK=64, DV=96, gate="vector", dtype="fp32", seed=52, gate_mean=3.0,
                    h0_std=0.1, dht_std=0.1)
    _report("narrow/fp32/wy7", tl.compare(tl.run_gpu(x, wy7=True), x))
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    xp = make_packed_inputs([70, 0, 130], H=2, gate="scalar", seed=53, cover=229)
    # narrow copies of the packed inputs: keys and values cut to 80 and 112
    for n in ("q", "k"):
        xp[n] = np.ascontiguousarray(xp[n][..., :80])
    for n in ("v", "dO"):
        xp[n] = np.ascontiguousarray(xp[n][..., :112])
    xp["h0"] = np.ascontiguousarray(xp["h0"][:, :, :80, :112])
    xp["dht"] = np.ascontiguousarray(xp["dht"][:, :, :80, :112])
    _report("narrow/packed", tl.compare_packed(tl.run_gpu_packed(xp), xp))


@pytest.mark.gpu
def test_packed_more_sequences_than_one_table_tile():
    """1500 sequences (the sequence tables are built in tiles of 1024 with a
    running carry), most of them short or empty, over 3000 tokens; the
    oracle checks every sequence of head 1."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs, packed_lengths
    x = make_packed_inputs(packed_lengths(3000, 1500, seed=7), H=2, gate="vector", seed=61,
                           gate_mean=3.0)
    _report("packed/1500", tl.compare_packed(tl.run_gpu_packed(x), x, heads=(1,)))


@pytest.mark.gpu
def test_many_heads_and_batch():
    """B = 4, H = 48 (768 state entries: wide scan launches), sampled heads."""
    _need_gpu()
    x = make_inputs(4, 192, 48, gate="scalar", dtype="bf16", seed=62, h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"B4H48/{pol}", tl.compare(tl.run_gpu(x, pol), x, heads=[(0, 0), (3, 47), (2, 17)]))


@pytest.mark.parametrize("gate", ["scalar", "vector"])
@pytest.mark.parametrize("T", [128, 150, 448])
def test_chunk_orders_small_chunk_counts(gate, T):
    """The per-chunk launches visit (chunk, head) items chunk-major in a
    cache-aware order (middle-out, ascending or descending by call); with
    2, 3 and 7 chunks and B * H = 6 every item must be visited exactly
    once under each order: both policies (the recompute backward's
    middle-out prep and local kernel, the forward's descending prep, the
    full-save backward's ascending xy and descending local kernel) and the
    seven-product local kernel."""
    _need_gpu()
    x = make_inputs(2, T, 3, gate=gate, dtype="bf16", seed=70 + T, h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"orders/{gate}/T{T}/{pol}", tl.compare(tl.run_gpu(x, pol), x))
    _report(f"orders/{gate}/T{T}/wy7", tl.compare(tl.run_gpu(x, wy7=True), x))


# ------------------------------------------------------ HIP graph capture

def _graph_case(x, policy, packed):
    """Forward + backward into preallocated outputs; returns a callable that
    launches both on the current stream, and the output tensors."""
    import torch
    import delta_rule_linear_gdr_amd as gdr
    d = tl.device_inputs(x)
    cu = torch.from_numpy(x["cu"]).to("cuda") if packed else None
    B, T, H = d["q"].shape[:3]
    ns = len(x["cu"]) - 1 if packed else B
    gate = "vector" if d["g"].dim() == 4 else "scalar"
    sv, sc = gdr.workspace_size(B, T, H, gate, "bf16", policy, n_seq=ns if packed else None)
    scratch = torch.empty(max(sc, 256), dtype=torch.uint8, device="cuda")
    saved = torch.empty(max(sv, 256), dtype=torch.uint8, device="cuda") if sv else None
    o = torch.empty_like(d["v"])
    ht = torch.empty((ns, H, 128, 128), dtype=torch.float32, device="cuda")
    out = dict(dq=torch.empty_like(d["q"]), dk=torch.empty_like(d["k"]), dv=torch.empty_like(d["v"]),
               dg=torch.empty_like(d["g"]), dbeta=torch.empty_like(d["beta"]),
               dh0=torch.empty((ns, H, 128, 128), dtype=torch.float32, device="cuda"))
    lib = gdr.load()
    desc = gdr._desc_from(d["q"], d["g"], d["v"])
    pol = gdr._policy(policy)
    P = gdr._ptr

    def launch():
        st = gdr._stream()
        fa = (P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["h0"]), P(o), P(ht),
              P(saved), P(scratch), scratch.numel(), st)
        ba = (P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["h0"]), P(d["dO"]),
              P(d["dht"]), P(saved), P(out["dq"]), P(out["dk"]), P(out["dv"]), P(out["dg"]),
              P(out["dbeta"]), P(out["dh0"]), P(scratch), scratch.numel(), st)
        import ctypes
        if packed:
            assert lib.gdr_fwd_varlen(ctypes.byref(desc), pol, P(cu), ns, *fa) == 0
            assert lib.gdr_bwd_varlen(ctypes.byref(desc), pol, P(cu), ns, *ba) == 0
        else:
            assert lib.gdr_fwd(ctypes.byref(desc), pol, *fa) == 0
            assert lib.gdr_bwd(ctypes.byref(desc), pol, *ba) == 0
    return launch, {"o": o, "ht": ht, **out}


@pytest.mark.gpu
@pytest.mark.parametrize("policy", ["recompute", "full_save"])
@pytest.mark.parametrize("packed", [False, True])
def test_graph_replay_matches_eager(policy, packed):
    """The forward + backward captured once in a HIP graph and replayed three
    times, with eager launches, output clearing and synchronizations between
    the replays: every replay equals the eager result bit for bit (the
    library allocates nothing, never synchronizes, clears memory with kernels
    and has no atomics)."""
    _need_gpu()
    import torch
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    if packed:
        x = make_packed_inputs([100, 0, 64, 131], H=2, gate="vector", seed=71, gate_mean=3.0)
    else:
        x = make_inputs(2, 200, 2, gate="vector", dtype="bf16", seed=72, gate_mean=3.0,
                        h0_std=0.1, dht_std=0.1)
    launch, outs = _graph_case(x, policy, packed)
    launch()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch()
    for rep in range(3):
        for t in outs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), f"replay {rep}: {n}"
        launch()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.gpu
def test_out_of_contract_decay_fails_loudly():
    """Every log decay -12 (a 16-token window spans 180, past the vector
    gate's contract of 160): the centred factors leave fp32 (exp(90)), and
    the output and gradients come out non-finite rather than finite and
    wrong."""
    _need_gpu()
    x = make_inputs(1, 256, 2, gate="vector", dtype="bf16", seed=3, h0_std=0.1, dht_std=0.1)
    x["g"] = np.full_like(x["g"], -12.0)
    assert tl.gate_check_bits(x["g"]) == tl.GATE_RANGE  # and gdr_gate_status says so (above)
    gpu = tl.run_gpu(x)
    for n in ("o", "dq", "dk", "dg"):
        assert not np.all(np.isfinite(gpu[n])), n


@pytest.mark.gpu
@pytest.mark.parametrize("policy", ["recompute", "full_save"])
def test_local_launch_forms_agree(policy):
    """The scalar-gate three-product local backward launched one workgroup
    per (chunk, head) (the form the like-for-like ablation times against the
    seven-product kernel) agrees with the persistent launch: the outputs the
    local kernel does not write bit for bit, its own outputs to fp32
    rounding (the two instantiations may order or fuse fp32 operations
    differently), and both meet the oracle's bar. Includes a ragged last
    chunk and a head count that leaves the persistent walk uneven."""
    _need_gpu()
    import delta_rule_linear_gdr_amd as gdr
    x = make_inputs(1, 1000, 5, gate="scalar", dtype="bf16", seed=21, gate_mean=4.0,
                    h0_std=0.1, dht_std=0.1)
    ref = tl.run_gpu(x, policy)
    prev = gdr.set_local_form("per_chunk")
    try:
        got = tl.run_gpu(x, policy)
    finally:
        gdr.set_local_form(prev)
    for n in ("o", "ht", "dh0"):
        assert np.array_equal(ref[n], got[n]), n
    diffs = {}
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        rel = np.linalg.norm(got[n] - ref[n]) / np.linalg.norm(ref[n])
        diffs[n] = (rel, float(np.max(np.abs(got[n] - ref[n]))))
        assert rel <= 1e-5, (n, rel)
    print("[launch forms] rel L2 / max abs: " +
          " ".join(f"{n}={a:.1e}/{b:.1e}" for n, (a, b) in diffs.items()), flush=True)
    _report(f"per_chunk/{policy}", tl.compare(got, x))


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["in_contract", "decay_-12", "one_positive", "one_nan",
                                  "strong_step", "scalar_positive", "ragged_in"])
def test_gate_status_reports_out_of_contract_decays(case):
    """The kernels' gate-check bits (gdr_gate_status) equal the plain
    statement of the contract (gdr_testlib.gate_check_bits) for the forward
    and the recompute backward, with no host synchronization inside either."""
    _need_gpu()
    import torch
    import delta_rule_linear_gdr_amd as gdr
    gate = "scalar" if case == "scalar_positive" else "vector"
    T = 200 if case == "ragged_in" else 256
    x = make_inputs(1, T, 2, gate=gate, dtype="bf16", seed=41, gate_mean=3.0)
    g = x["g"].copy()
    if case == "decay_-12":
        g[:] = -12.0
    elif case == "one_positive":
        g[0, 100, 1, 5] = 0.25
    elif case == "one_nan":
        g[0, 7, 0, 3] = np.nan
    elif case == "strong_step":
        g[0, 130, 1, 77] = -170.0  # row 2 of chunk 2's first window
    elif case == "scalar_positive":
        g[0, 33, 1] = 0.5
    x["g"] = g
    want = tl.gate_check_bits(g)
    d = tl.device_inputs(x)
    for policy in ("recompute", "full_save"):
        _, sc = gdr.workspace_size(1, T, 2, gate, "bf16", policy)
        scratch = torch.empty(sc, dtype=torch.uint8, device="cuda")
        gdr.gdr_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], policy=policy,
                    scratch=scratch)
        got_f = int(gdr.gate_status(d["q"], d["g"], d["v"], scratch).item())
        assert got_f == want, (policy, "forward", got_f, want)
        if policy == "recompute":
            gdr.gdr_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["dO"], None,
                        scratch=scratch)
            got_b = int(gdr.gate_status(d["q"], d["g"], d["v"], scratch).item())
            assert got_b == want, ("backward", got_b, want)
    print(f"[gate status] {case}: {want}", flush=True)


@pytest.mark.gpu
@pytest.mark.parametrize("gate", ["scalar", "vector"])
@pytest.mark.parametrize("dk,dv", [(128, 160), (80, 160), (64, 300)])
def test_value_widths_above_128(gate, dk, dv):
    """Value widths above 128 (the pages' extended tests use a value width of
    160) run as 128-wide value blocks whose key-side gradients are summed:
    two batch entries, a ragged last chunk, nonzero states, both policies."""
    _need_gpu()
    x = make_inputs(2, 100, 2, DK=dk, DV=dv, gate=gate, dtype="bf16", seed=54,
                    gate_mean=4.0 if gate == "scalar" else 3.0, h0_std=0.1, dht_std=0.1)
    for pol in ("recompute", "full_save"):
        _report(f"wide/{gate}/{dk}x{dv}/{pol}", tl.compare(tl.run_gpu(x, pol), x))


@pytest.mark.gpu
def test_value_width_160_fp32_wy7_deltanet_and_packed():
    """Value width 160 with fp32 storage and the seven-product producer, with
    no gate (DeltaNet), and in a packed batch with a tail of tokens outside
    every sequence."""
    _need_gpu()
    x = make_inputs(1, 150, 2, DK=96, DV=160, gate="vector", dtype="fp32", seed=55, gate_mean=3.0,
                    h0_std=0.1, dht_std=0.1)
    _report("wide/fp32/wy7", tl.compare(tl.run_gpu(x, wy7=True), x))
    xn = make_inputs(1, 130, 2, DK=128, DV=160, gate="scalar", dtype="bf16", seed=56,
                     h0_std=0.1, dht_std=0.1)
    xn["g"] = np.zeros_like(xn["g"])
    _report("wide/deltanet", tl.compare(tl.run_gpu(xn, nogate=True), xn))
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    xp = make_packed_inputs([70, 0, 130], H=2, gate="scalar", seed=57, cover=241)
    rng = np.random.default_rng(58)
    # value width 160: the packed inputs' 128 value columns and 32 more
    for n in ("v", "dO"):
        extra = np.asarray(xp[n][..., :32])[..., ::-1]
        xp[n] = np.ascontiguousarray(np.concatenate([xp[n], extra], axis=-1))
    for n in ("h0", "dht"):
        xp[n] = np.ascontiguousarray(np.concatenate(
            [xp[n], (0.1 * rng.standard_normal(xp[n].shape[:-1] + (32,))).astype(np.float32)
             .astype(np.float64)], axis=-1))
    _report("wide/packed", tl.compare_packed(tl.run_gpu_packed(xp), xp))


@pytest.mark.gpu
@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_packed_value_blocks_both_policies(gate):
    """A packed batch at value width 200 (two value blocks: 128 + 72) with an
    empty sequence, a ragged one and a tail of tokens outside every sequence,
    under both policies (the full-save area holds one block's set per block)."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    xp = make_packed_inputs([90, 0, 150], H=2, gate=gate, seed=63, gate_mean=3.0, cover=270)
    rng = np.random.default_rng(64)
    # value width 200: the packed inputs' 128 value columns and 72 more
    for n in ("v", "dO"):
        extra = np.asarray(xp[n][..., :72])[..., ::-1]
        xp[n] = np.ascontiguousarray(np.concatenate([xp[n], extra], axis=-1))
    for n in ("h0", "dht"):
        xp[n] = np.ascontiguousarray(np.concatenate(
            [xp[n], (0.1 * rng.standard_normal(xp[n].shape[:-1] + (72,))).astype(np.float32)
             .astype(np.float64)], axis=-1))
    for pol in ("recompute", "full_save"):
        _report(f"packed/200/{gate}/{pol}", tl.compare_packed(tl.run_gpu_packed(xp, pol), xp))


@pytest.mark.gpu
def test_deltanet_packed_narrow_with_tail():
    """DeltaNet (no gate) over a packed batch at widths 80/112 with a tail of
    tokens outside every sequence, under both policies: the zero-gate
    workspace, the padded copies and the packed tables together."""
    _need_gpu()
    from delta_rule_linear_gdr_amd.inputs import make_packed_inputs
    x = make_packed_inputs([70, 0, 130, 1], H=2, gate="scalar", seed=65, cover=230)
    x["g"] = np.zeros_like(x["g"])
    for n in ("q", "k"):
        x[n] = np.ascontiguousarray(x[n][..., :80])
    for n in ("v", "dO"):
        x[n] = np.ascontiguousarray(x[n][..., :112])
    for n in ("h0", "dht"):
        x[n] = np.ascontiguousarray(x[n][:, :, :80, :112])
    for pol in ("recompute", "full_save"):
        got = tl.run_gpu_packed(x, pol, nogate=True)
        assert "dg" not in got
        _report(f"deltanet/packed/80x112/{pol}", tl.compare_packed(got, x))


# ------------------------------------------------------- two-level walks

@pytest.mark.gpu
@pytest.mark.parametrize("B,T,H,gate,dtype", [
    (1, 8192, 4, "scalar", "bf16"),   # forward and full-save reverse 5 segments; recompute pair one level
    (1, 6144, 2, "vector", "bf16"),   # 4 segments of 24 chunks, every launch
    (2, 7000, 1, "scalar", "fp32"),   # ragged last chunk, 5 segments of at most 22 chunks
])
def test_two_level_walks_match_oracle_and_one_level(B, T, H, gate, dtype):
    """Walks cut into segments (entry-to-exit maps formed for all segments at
    once, entry states chained through them, then every segment walked from
    its own entry state) against the oracle, with nonzero h0 and dht, under
    both policies; and against the same calls with one-level walks."""
    _need_gpu()
    import delta_rule_linear_gdr_amd as gdr
    x = make_inputs(B, T, H, gate=gate, dtype=dtype, seed=71, gate_mean=3.0 if gate == "vector" else 4.0,
                    h0_std=0.1, dht_std=0.1)
    heads = None if B * H <= 2 else [(0, 0), (0, H - 1)]
    for pol in ("recompute", "full_save"):
        two = tl.run_gpu(x, pol)
        prev = gdr.set_walk_levels("one")
        try:
            one = tl.run_gpu(x, pol)
        finally:
            gdr.set_walk_levels(prev)
        _report(f"two-level {B}x{T}x{H}/{gate}/{dtype}/{pol}", tl.compare(two, x, heads=heads))
        tl.compare(one, x, heads=heads)
        # the two forms agree far inside the bar
        for n in two:
            den = np.linalg.norm(one[n])
            if den > 0:
                assert np.linalg.norm(two[n] - one[n]) / den < 4e-3, n


@pytest.mark.gpu
def test_two_level_walks_deltanet_and_seven_product():
    """Two-level walks with no gate and with the seven-product backward."""
    _need_gpu()
    x = make_inputs(1, 6144, 2, gate="scalar", dtype="bf16", seed=72, h0_std=0.1, dht_std=0.1)
    xn = dict(x)
    xn["g"] = np.zeros_like(x["g"])
    _report("two-level deltanet", tl.compare(tl.run_gpu(xn, nogate=True), xn))
    _report("two-level wy7", tl.compare(tl.run_gpu(x, "full_save", wy7=True), x))
