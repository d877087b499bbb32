"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the library through its Python binding, run the CPU oracle on the same
values, and apply the acceptance rule.

Acceptance (ReWY paper, Sec. 4.5 "Numerical validation": 0.8% relative for
ordinary outputs and gradients, 2% for gate and beta gradients, a maximum
absolute threshold for near-zero references, all values finite), read per
tensor: if max|ref| <= 1e-6 the maximum absolute error must be <= 1e-6,
otherwise ||x - ref||_2 / ||ref||_2 must be within the tolerance.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = {"o": 0.008, "ht": 0.008, "dq": 0.008, "dk": 0.008, "dv": 0.008, "dh0": 0.008,
       "dg": 0.02, "dbeta": 0.02}
NEAR_ZERO = 1e-6


def check(name, got, ref, tol=None):
    tol = TOL[name] if tol is None else tol
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if np.max(np.abs(ref), initial=0.0) <= NEAR_ZERO:
        err = np.max(np.abs(got - ref), initial=0.0)
        assert err <= NEAR_ZERO, f"{name}: near-zero reference, max abs err {err:.3e}"
        return err
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= tol, f"{name}: rel L2 {rel:.5f} > {tol}"
    return rel


def to_dev(x, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


def device_inputs(x):
    import torch
    dt = torch_dtype(x["dtype"])
    d = {n: to_dev(x[n], dt) for n in ("q", "k", "v", "beta", "dO")}
    d["g"] = to_dev(x["g"], torch.float32)
    d["h0"] = to_dev(x["h0"], torch.float32)
    d["dht"] = to_dev(x["dht"], torch.float32)
    return d


def run_gpu(x, policy="recompute", wy7=False, use_h0=True, use_dht=True, nogate=False):
    """Forward + backward on the device; returns numpy float64 results.
    nogate: call with g = None (DeltaNet; x["g"] must then be all zero)."""
    import torch
    import delta_rule_linear_gdr_amd as gdr
    d = device_inputs(x)
    h0 = d["h0"] if use_h0 else None
    dht = d["dht"] if use_dht else None
    g = None if nogate else d["g"]
    o, ht, saved = gdr.gdr_fwd(d["q"], d["k"], d["v"], g, d["beta"], h0, policy=policy)
    fn = gdr.gdr_bwd_wy7 if wy7 else gdr.gdr_bwd
    gr = fn(d["q"], d["k"], d["v"], g, d["beta"], h0, d["dO"], dht, saved=saved,
            policy=policy)
    torch.cuda.synchronize()
    out = {"o": o, "ht": ht, **gr}
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items()
            if t is not None}


def oracle_heads(x, heads=None, threads=None):
    """Oracle forward + backward restricted to (b, h) pairs (all if None).
    Returns per-tensor arrays stacked along a leading 'pair' axis."""
    B, T, H, _ = x["q"].shape
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    res = {n: [] for n in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0")}
    for b, h in pairs:
        sl = lambda a: a[b:b + 1, :, h:h + 1]  # noqa: E731
        st = lambda a: a[b:b + 1, h:h + 1]     # noqa: E731
        o, ht = oracle.token_fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]),
                                 sl(x["beta"]), st(x["h0"]), threads=threads)
        gr = oracle.token_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                              st(x["h0"]), sl(x["dO"]), st(x["dht"]), threads=threads)
        res["o"].append(o)
        res["ht"].append(ht)
        for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
            res[n].append(gr[n])
    return pairs, res


def select_heads(gpu, pairs):
    """Restrict full GPU results to the oracle's (b, h) pairs, same stacking."""
    out = {}
    for n, a in gpu.items():
        if a is None:
            continue
        if n in ("ht", "dh0"):
            out[n] = [a[b:b + 1, h:h + 1] for b, h in pairs]
        else:
            out[n] = [a[b:b + 1, :, h:h + 1] for b, h in pairs]
    return out


def compare(gpu, x, heads=None, names=None, report=None):
    pairs, ref = oracle_heads(x, heads)
    got = select_heads(gpu, pairs)
    errs = {}
    for n in names or ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        if n not in got:
            continue
        errs[n] = check(n, np.concatenate(got[n]), np.concatenate(ref[n]))
    if report is not None:
        report.update(errs)
    return errs


def compare_all_heads(gpu, x, report=None):
    """Every (b, h) pair of the workload: one threaded oracle call for the
    whole problem, then the acceptance rule per tensor over all heads and,
    so that an error confined to one head or batch entry cannot hide in the
    total, per tensor on every (b, h) pair on its own."""
    o, ht = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    ref = oracle.token_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["dO"], x["dht"])
    ref.update(o=o, ht=ht)
    B, _, H = x["q"].shape[:3]
    errs = {}
    for n in ("o", "ht", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        if n not in gpu:
            continue
        errs[n] = check(n, gpu[n], ref[n])
        worst = 0.0
        for b in range(B):
            for h in range(H):
                if n in ("ht", "dh0"):
                    g_, r_ = gpu[n][b, h], ref[n][b, h]
                else:
                    g_, r_ = gpu[n][b, :, h], ref[n][b, :, h]
                e = check(n, g_, r_)
                worst = max(worst, e)
        errs[n + "_worst_head"] = worst
    if report is not None:
        report.update(errs)
    return errs


# ---------------------------------------------------- packed (varlen) batches

SENTINEL = 7.0  # prefilled into o and the gradient outputs; tokens of no sequence keep it


def run_gpu_packed(x, policy="recompute", nogate=False):
    """Packed forward + backward (cu_seqlens) on the device; numpy float64.
    nogate: call with g = None (DeltaNet; x["g"] must then be all zero)."""
    import torch
    import delta_rule_linear_gdr_amd as gdr
    d = device_inputs(x)
    g = None if nogate else d["g"]
    cu = torch.from_numpy(x["cu"]).to("cuda")
    o, ht, saved = gdr.gdr_fwd(d["q"], d["k"], d["v"], g, d["beta"], d["h0"],
                               policy=policy, cu_seqlens=cu, o=torch.full_like(d["v"], SENTINEL))
    out = {n: torch.full_like(d[s], SENTINEL) for n, s in
           (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta"))
           if not (nogate and n == "dg")}
    out["dh0"] = torch.empty_like(d["h0"])
    gr = gdr.gdr_bwd(d["q"], d["k"], d["v"], g, d["beta"], d["h0"], d["dO"], d["dht"],
                     saved=saved, policy=policy, out=out, cu_seqlens=cu)
    torch.cuda.synchronize()
    res = {"o": o, "ht": ht, **gr}
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in res.items() if t is not None}


def oracle_packed(x, heads=None):
    """Oracle per (sequence, head): each sequence is its own problem with its
    own h0 and dht. An empty sequence passes its state through (ht = h0,
    dh0 = dht), which needs no oracle call."""
    cu = x["cu"]
    H = x["q"].shape[2]
    heads = range(H) if heads is None else heads
    ref = {}
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        for h in heads:
            sl = lambda t: t[:, a:b, h:h + 1]       # noqa: E731
            st = lambda t: t[i:i + 1, h:h + 1]      # noqa: E731
            if b == a:
                ref[i, h] = {"ht": st(x["h0"]), "dh0": st(x["dht"])}
                continue
            o, ht = oracle.token_fwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]),
                                     sl(x["beta"]), st(x["h0"]))
            gr = oracle.token_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                                  st(x["h0"]), sl(x["dO"]), st(x["dht"]))
            ref[i, h] = {"o": o, "ht": ht, **gr}
    return ref


def compare_packed(gpu, x, heads=None, report=None):
    """Per-tensor acceptance over the covered tokens of the chosen heads, and
    the outputs of tokens outside every sequence left untouched."""
    cu = x["cu"]
    ref = oracle_packed(x, heads)
    got_all, ref_all = {}, {}
    for (i, h), r in ref.items():
        a, b = int(cu[i]), int(cu[i + 1])
        for n, arr in r.items():
            if n not in gpu:
                continue
            g = gpu[n][i:i + 1, h:h + 1] if n in ("ht", "dh0") else gpu[n][:, a:b, h:h + 1]
            got_all.setdefault(n, []).append(g.ravel())
            ref_all.setdefault(n, []).append(np.asarray(arr).ravel())
    errs = {n: check(n, np.concatenate(got_all[n]), np.concatenate(ref_all[n]))
            for n in got_all}
    tail = int(cu[-1])
    for n in ("o", "dq", "dk", "dv", "dg", "dbeta"):
        if n not in gpu:
            continue
        assert np.all(gpu[n][:, tail:] == SENTINEL), f"{n}: tokens past the last sequence written"
    if report is not None:
        report.update(errs)
    return errs


# ---------------------------------------------------------------- gate check

GATE_POSITIVE, GATE_RANGE, GATE_NONFINITE = 1, 2, 4


def gate_check_bits(g, T=None, window=16, chunk=64, limit=160.0):
    """The contract of the log decays, stated plainly: bit 1 if any log decay
    is above 0, bit 4 if any is NaN or infinite, and (per-channel gates,
    g [B,T,H,DK]) bit 2 if, within any 64-token chunk, the chunk-local
    cumulative log decay of some channel spans more than `limit` over one
    16-token window of the chunk. A ragged chunk's missing rows count as
    zero decay."""
    g = np.asarray(g, dtype=np.float64)
    bits = 0
    if np.any(g > 0):
        bits |= GATE_POSITIVE
    if not np.all(np.isfinite(g)):
        bits |= GATE_NONFINITE
    if g.ndim == 4:
        B, T_, H, DK = g.shape
        for c0 in range(0, T_, chunk):
            G = np.cumsum(np.nan_to_num(g[:, c0:c0 + chunk], nan=0.0, posinf=0.0, neginf=0.0), axis=1)
            n = G.shape[1]
            if n < chunk:  # ragged: missing rows keep the last cumulative value
                G = np.concatenate([G, np.repeat(G[:, -1:], chunk - n, axis=1)], axis=1)
            for w0 in range(0, chunk, window):
                Gw = G[:, w0:w0 + window]
                if np.any(Gw.max(axis=1) - Gw.min(axis=1) > limit):
                    bits |= GATE_RANGE
    return bits
