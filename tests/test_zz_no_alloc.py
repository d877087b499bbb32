"""gdr_bwd_noalloc (the backward whose scratch is the library's fixed device
array, for callers that cannot allocate) against gdr_bwd with a caller
workspace, through the C ABI: two calls in a row on one device, the second
on a smaller problem, each equal to gdr_bwd bit for bit (same kernels, same
arithmetic; only the workspace address differs)."""
import ctypes

import numpy as np
import pytest

from delta_rule_linear_gdr_amd.inputs import make_inputs
from tests import gdr_testlib as tl

pytestmark = pytest.mark.gpu


def _backward_pair(x, policy):
    import torch
    import delta_rule_linear_gdr_amd as gdr
    d = tl.device_inputs(x)
    lib = gdr.load()
    desc = gdr._desc_from(d["q"], d["g"], d["v"])
    pol = gdr._policy(policy)
    P = gdr._ptr
    B, T, H = d["q"].shape[:3]
    gate = "vector" if d["g"].dim() == 4 else "scalar"
    sv, sc = gdr.workspace_size(B, T, H, gate, "bf16", policy)
    assert sc <= lib_max(), (sc, lib_max())
    scratch = torch.empty(max(sc, 256), dtype=torch.uint8, device="cuda")
    saved = None
    if sv:
        saved = torch.empty(sv, dtype=torch.uint8, device="cuda")
        o = torch.empty_like(d["v"])
        assert lib.gdr_fwd(ctypes.byref(desc), pol, P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]),
                           P(d["beta"]), P(d["h0"]), P(o), None, P(saved), P(scratch),
                           scratch.numel(), gdr._stream()) == 0

    def outs():
        return dict(dq=torch.full_like(d["q"], float("nan")), dk=torch.full_like(d["k"], float("nan")),
                    dv=torch.full_like(d["v"], float("nan")), dg=torch.full_like(d["g"], float("nan")),
                    dbeta=torch.full_like(d["beta"], float("nan")),
                    dh0=torch.full((B, H, 128, 128), float("nan"), dtype=torch.float32, device="cuda"))
    ref, got = outs(), outs()
    common = (P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["h0"]), P(d["dO"]),
              P(d["dht"]), P(saved))
    rc = lib.gdr_bwd(ctypes.byref(desc), pol, *common, P(ref["dq"]), P(ref["dk"]), P(ref["dv"]),
                     P(ref["dg"]), P(ref["dbeta"]), P(ref["dh0"]), P(scratch), scratch.numel(),
                     gdr._stream())
    assert rc == 0, lib.gdr_last_error()
    rc = lib.gdr_bwd_noalloc(ctypes.byref(desc), pol, *common, P(got["dq"]), P(got["dk"]),
                             P(got["dv"]), P(got["dg"]), P(got["dbeta"]), P(got["dh0"]),
                             gdr._stream())
    assert rc == 0, lib.gdr_last_error()
    torch.cuda.synchronize()
    return ref, got


def lib_max():
    return 64 << 20


def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_noalloc_equals_gdr_bwd_on_two_calls():
    _need_gpu()
    import torch
    cases = [
        # the largest recompute problem of the pages' shapes that fits the array
        (make_inputs(1, 2048, 8, gate="scalar", dtype="bf16", seed=11, gate_mean=4.0,
                     h0_std=0.1, dht_std=0.1), "recompute"),
        # then a smaller one, ragged, vector gate, full save
        (make_inputs(1, 700, 3, gate="vector", dtype="bf16", seed=12, gate_mean=3.0,
                     h0_std=0.1, dht_std=0.1), "full_save"),
    ]
    for i, (x, policy) in enumerate(cases):
        print(f"[noalloc] call {i}: {x['q'].shape} {policy}", flush=True)
        ref, got = _backward_pair(x, policy)
        for n in ref:
            assert torch.isfinite(ref[n]).all(), n
            assert torch.equal(ref[n], got[n]), f"call {i}: {n} differs"
        # and, for the record, the oracle's bar on the no-alloc result
        res = {n: t.float().cpu().numpy().astype(np.float64) for n, t in got.items()}
        errs = tl.compare(res, x, names=("dq", "dk", "dv", "dg", "dbeta", "dh0"))
        print(f"[noalloc] call {i}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)


def test_noalloc_with_two_level_walks():
    """A problem whose recompute backward walks in segments, (1, 8192, 2):
    the segment summaries and entry states live in the fixed array too, and
    the result equals gdr_bwd's bit for bit."""
    _need_gpu()
    import torch
    x = make_inputs(1, 8192, 2, gate="scalar", dtype="bf16", seed=13, gate_mean=4.0,
                    h0_std=0.1, dht_std=0.1)
    print(f"[noalloc] two-level: {x['q'].shape} recompute", flush=True)
    ref, got = _backward_pair(x, "recompute")
    for n in ref:
        assert torch.isfinite(ref[n]).all(), n
        assert torch.equal(ref[n], got[n]), f"{n} differs"
