"""Seeded synthetic inputs for chunkwise gated delta-rule attention.

This module holds the input recipe only -- random draws, per-token feature
normalisation, the gate/weight activations that produce the operator's inputs,
and rounding to the storage dtype. It contains none of the operator's
arithmetic, and it is the one module that both the GPU path's tests/bench and
the CPU oracle's callers use.

Recipe (ReWY paper App. G.3 "Numerical coverage": feature-normalised Gaussian
queries/keys, Gaussian values and output adjoints, query scale, Gaussian
states scaled by 0.1; log gates from a log-sigmoid; weights in (0, 1)):
  numpy.random.default_rng(seed), float64 draws in this order:
    q_raw, k_raw, v ~ N(0, 1)                       [B,T,H,DK|DV]
    gate_pre ~ N(gate_mean, 1)                      [B,T,H] or [B,T,H,DK]
    beta_pre ~ N(0, 1)                              [B,T,H]
    dO ~ N(0, 1)                                    [B,T,H,DV]
    h0  = h0_std  * N(0, 1)                         [B,H,DK,DV]  (only if h0_std > 0)
    dht = dht_std * N(0, 1)                         [B,H,DK,DV]  (only if dht_std > 0)
    GDN2 only (gate "gdn2": per-key-channel gate_pre as for "vector"):
    ers_pre ~ N(0, 1) [B,T,H,DK], wrt_pre ~ N(0, 1) [B,T,H,DV]
  q = q_raw / |q_raw| / sqrt(DK);  k = k_raw / |k_raw|   (per token and head)
  g = log_sigmoid(gate_pre)  (stored fp32);  beta = sigmoid(beta_pre)
  GDN2: erase ers = sigmoid(ers_pre), write wrt = sigmoid(wrt_pre) (weights in
  (0, 1) per channel, like beta; the paper's main experiments keep the
  erase/write weights in the input format, Sec. 3.5)
  q, k, v, beta, dO (and ers, wrt) are rounded to the storage dtype (bf16:
  round-to-nearest-even through fp32); g, h0, dht are fp32.
Every returned array is float64 holding exactly the rounded values, so a
reference computed from them sees the same numbers as the device.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def round_fp32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest-even, via fp32), returned as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return round_fp32(x)
    raise ValueError(dtype)


@dataclass
class Workload:
    """A named synthetic workload (shape + distributions)."""
    name: str
    gate: str          # "scalar" (GDN), "vector" (KDA) or "gdn2"
    B: int
    T: int
    H: int
    dtype: str = "bf16"
    DK: int = 128
    DV: int = 128
    gate_mean: float = 4.0
    h0_std: float = 0.0
    dht_std: float = 0.0
    seed: int = 0

    def make(self) -> dict:
        return make_inputs(self.B, self.T, self.H, self.DK, self.DV, self.gate, self.dtype,
                           self.seed, self.gate_mean, self.h0_std, self.dht_std)


# The parity and benchmark workloads: GDN at (1,512,4) fp32, (1,2048,16) and
# (1,8192,16) bf16; KDA at (2,2048,16) and (1,8192,16) bf16 with h0 ~ 0.1 N(0,1);
# and GDN2 at the headline shape, drawn like KDA's with both gates.
# The six (B, T, H) shapes of the pages' evaluation (Eq. 4 of the paper page,
# listed in the onedev.kr summary's "How to use"), C = 64, d_k = d_v = 128.
SHAPES6 = ((1, 512, 4), (1, 2048, 4), (1, 8192, 4), (1, 2048, 16), (2, 2048, 16), (1, 8192, 16))

WORKLOADS = {
    "gdn_1x512x4_fp32": Workload("gdn_1x512x4_fp32", "scalar", 1, 512, 4, "fp32"),
    "gdn_1x2048x16": Workload("gdn_1x2048x16", "scalar", 1, 2048, 16),
    "gdn_1x8192x16": Workload("gdn_1x8192x16", "scalar", 1, 8192, 16),
    "kda_2x2048x16": Workload("kda_2x2048x16", "vector", 2, 2048, 16, gate_mean=3.0),
    "kda_1x8192x16": Workload("kda_1x8192x16", "vector", 1, 8192, 16, gate_mean=3.0,
                              h0_std=0.1),
    "gdn2_1x8192x16": Workload("gdn2_1x8192x16", "gdn2", 1, 8192, 16, gate_mean=3.0,
                               h0_std=0.1),
}


def make_inputs(B, T, H, DK=128, DV=128, gate="scalar", dtype="bf16", seed=0,
                gate_mean=4.0, h0_std=0.0, dht_std=0.0) -> dict:
    rng = np.random.default_rng(seed)
    q_raw = rng.standard_normal((B, T, H, DK))
    k_raw = rng.standard_normal((B, T, H, DK))
    v = rng.standard_normal((B, T, H, DV))
    if gate not in ("scalar", "vector", "gdn2"):
        raise ValueError(f"unknown gate {gate!r}")
    gshape = (B, T, H) if gate == "scalar" else (B, T, H, DK)
    gate_pre = rng.standard_normal(gshape) + gate_mean
    beta_pre = rng.standard_normal((B, T, H))
    dO = rng.standard_normal((B, T, H, DV))
    h0 = h0_std * rng.standard_normal((B, H, DK, DV)) if h0_std > 0 else np.zeros((B, H, DK, DV))
    dht = dht_std * rng.standard_normal((B, H, DK, DV)) if dht_std > 0 else np.zeros((B, H, DK, DV))
    extra = {}
    if gate == "gdn2":
        ers_pre = rng.standard_normal((B, T, H, DK))
        wrt_pre = rng.standard_normal((B, T, H, DV))
        extra["ers"] = round_to(1.0 / (1.0 + np.exp(-ers_pre)), dtype)
        extra["wrt"] = round_to(1.0 / (1.0 + np.exp(-wrt_pre)), dtype)
    qn = np.linalg.norm(q_raw, axis=-1, keepdims=True)
    kn = np.linalg.norm(k_raw, axis=-1, keepdims=True)
    q = q_raw / np.maximum(qn, 1e-30) / np.sqrt(DK)
    k = k_raw / np.maximum(kn, 1e-30)
    g = -np.logaddexp(0.0, -gate_pre)           # log_sigmoid
    beta = 1.0 / (1.0 + np.exp(-beta_pre))       # sigmoid
    return dict(
        q=round_to(q, dtype), k=round_to(k, dtype), v=round_to(v, dtype),
        g=round_fp32(g), beta=round_to(beta, dtype), dO=round_to(dO, dtype),
        h0=round_fp32(h0), dht=round_fp32(dht),
        gate=gate, dtype=dtype, **extra,
    )


def packed_lengths(total: int, n: int, seed: int = 0) -> list[int]:
    """Lengths of n sequences packed into `total` tokens: n - 1 cut points
    drawn uniformly (with replacement) from [0, total] and sorted, so the mix
    holds short, long and occasionally empty sequences."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.integers(0, total + 1, size=max(n - 1, 0)))
    edges = np.concatenate([[0], cuts, [total]])
    return [int(x) for x in np.diff(edges)]


def make_packed_inputs(lengths, H, gate="scalar", dtype="bf16", seed=0, gate_mean=4.0,
                       state_std=0.1, cover=None) -> dict:
    """A packed variable-length batch: the sequences of `lengths` laid end to
    end in one row of `cover` tokens (default: their sum; more leaves a tail
    that belongs to no sequence). Token inputs follow make_inputs(1, cover, H,
    seed=seed); then numpy.random.default_rng(seed + 1) draws the per-sequence
    states h0 and dht = state_std * N(0, 1), [n, H, DK, DV] each, rounded to
    fp32. cu holds the n + 1 int64 token offsets."""
    lengths = [int(x) for x in lengths]
    T = sum(lengths) if cover is None else int(cover)
    assert T >= sum(lengths)
    x = make_inputs(1, T, H, gate=gate, dtype=dtype, seed=seed, gate_mean=gate_mean)
    n = len(lengths)
    rng = np.random.default_rng(seed + 1)
    x["h0"] = round_fp32(state_std * rng.standard_normal((n, H, 128, 128)))
    x["dht"] = round_fp32(state_std * rng.standard_normal((n, H, 128, 128)))
    x["cu"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return x
