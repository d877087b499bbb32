"""The roofline accounting that bench.py reports, checked on the CPU.

Every figure in bench.py's byte and FLOP tables is recounted here from a
plain list of the tensors each kernel reads and writes (shape and stored
type, as the C ABI and the kernels store them) and from the dense products
of the hot-path steps. The committed counter summaries' "algorithmic bytes
per launch" columns must equal the same table times the (chunk, head) count
of their workload.
"""
import json
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CH, D = 64, 128
BF16, F32 = 2, 4


def nbytes(*shape_and_size):
    *shape, size = shape_and_size
    n = size
    for x in shape:
        n *= x
    return n


def gate_bytes(gate):
    # log decay and its gradient: one fp32 per token (scalar gate) or per
    # token and key channel (vector gate)
    return nbytes(CH, F32) if gate == "scalar" else nbytes(CH, D, F32)


def kernel_tensors(gate):
    """Per (chunk, head): the tensors each kernel reads and writes once."""
    tok = nbytes(CH, D, BF16)          # a 64-token x 128-channel bf16 tile
    state = nbytes(D, D, BF16)         # a stored 128 x 128 state (h_c, dh_c)
    tri = nbytes(CH, CH, BF16)         # A, A^T, H^T
    gn = nbytes(D, F32)                # exp of the chunk's total log decay, per key channel
    g = gate_bytes(gate)
    if gate == "gdn2":
        # the erase (64 x 128 keys) and write (64 x 128 values) gates in bf16
        # take beta's place, and their gradients dbeta's
        inputs = [tok] * 4 + [g, tok, tok]   # q, k, v, dO, g, erase, write
        grads = [tok] * 3 + [g, tok, tok]    # dq, dk, dv, dg, derase, dwrite
    else:
        beta = nbytes(CH, BF16)
        inputs = [tok] * 4 + [g, beta]     # q, k, v, dO, g, beta
        grads = [tok] * 3 + [g, beta]      # dq, dk, dv, dg, dbeta
    return {
        # writes -W, K~, U, X (64 x 128 each), Y (128 x 128), A^T, gn
        "prep": inputs + [tok] * 4 + [state, tri, gn],
        # forward walk reads -W, K~ (as K~^T), U, gn and writes h, R
        "scan_fwd": [tok, tok, tok, gn, state, tok],
        # reverse walk reads K~, -W (as -W^T), X, Y, gn and writes dh, Rbar
        "scan_bwd": [tok, tok, tok, state, gn, state, tok],
        # both walks in one launch read -W, K~ and gn, counted once
        "scan_pair": [tok, tok, gn] + [tok, state, tok] + [tok, state, state, tok],
        # reads q, k, v, dO, g, beta, R, Rbar, h, dh, A^T; writes the gradients
        "bwd_local": inputs + [tok, tok, state, state, tri] + grads,
        "bwd_local_wy7": inputs + [tok, tok, state, state, tri, tri] + grads,
        # reads H^T, Q_g^T, dO; writes X, Y
        "xy": [tri, tok, tok, tok, state],
    }


@pytest.mark.parametrize("gate", ["scalar", "vector", "gdn2"])
def test_kernel_bytes_match_the_tensor_lists(gate):
    work = bench.kernel_work(gate)
    for name, tensors in kernel_tensors(gate).items():
        assert work[name][0] == sum(tensors), name


def test_bwd_local_bytes_per_chunk_head():
    # the figure the dominant-kernel roofline is quoted on
    assert bench.kernel_work("scalar")["bwd_local"][0] == 221952
    assert bench.kernel_work("scalar")["bwd_local"][0] * 2048 == 454557696


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_whole_path_bytes_per_token_head(gate):
    # the operator's own inputs and outputs per token and head
    row = D * BF16
    g = 4 if gate == "scalar" else D * 4
    fwd = 3 * row + g + BF16 + row                    # q, k, v, g, beta -> o
    bwd = 4 * row + g + BF16 + 3 * row + g + BF16     # q, k, v, dO, g, beta -> dq, dk, dv, dg, dbeta
    # the full-save area per token-head: A row (64 bf16), W row, R row, and a
    # 64th of the chunk's stored 128 x 128 bf16 state
    saved = CH * BF16 + row + row + D * D * BF16 // CH
    assert saved == 1152
    t = bench.PATH_BYTES_PER_TOKEN_HEAD
    assert t[(gate, "fwd_R")] == fwd
    assert t[(gate, "fwd_A")] == fwd + saved
    assert t[(gate, "bwd_R")] == bwd
    assert t[(gate, "bwd_A")] == bwd + saved


def test_gdn2_whole_path_bytes_per_token_head():
    # GDN2: a per-key fp32 log decay, and per-key erase and per-value write
    # gates in bf16 in place of beta (their gradients likewise)
    row = D * BF16
    g = D * 4
    fwd = 3 * row + g + 2 * row + row                 # q, k, v, g, erase, write -> o
    bwd = 4 * row + g + 2 * row + 3 * row + g + 2 * row
    t = bench.PATH_BYTES_PER_TOKEN_HEAD
    assert (t[("gdn2", "fwd_R")], t[("gdn2", "bwd_R")]) == (fwd, bwd) == (2048, 3840)


def test_path_flops_are_the_launched_kernels_flops():
    w = bench.kernel_work("scalar")
    f = bench.PATH_FLOPS_PER_CHUNK_HEAD
    # recompute backward: prep -> both walks -> local kernel
    assert f["bwd_R"] == w["prep"][1] + w["scan_pair"][1] + w["bwd_local"][1]
    # full-save backward: xy -> reverse walk -> local kernel
    assert f["bwd_A"] == w["xy"][1] + w["scan_bwd"][1] + w["bwd_local"][1]


def test_flops_follow_the_hot_path_products():
    unit = 2 * CH * CH * D                 # one 64 x 64 x 128 product
    assert bench.M == unit
    # forward: L = strict_lower(E Y^T) (1), W = A E and U = A Z (2), the solve,
    # the walk's W S and K~^T R (2 + 2), the output's Q_g S (2) and
    # H = lower(Q_g Y^T) (1) with H R (1)
    fwd = unit * (1 + 2 + 4 + 2 + 1 + 1) + CH ** 3 // 3
    assert bench.PATH_FLOPS_PER_CHUNK_HEAD["fwd_R"] == fwd
    # the local kernel: the three ReWY products A^T Rbar (1), P R^T (1),
    # P h^T (2); Gram elimination's four contractions (4) and Hbar (1); the
    # state-direct Obar h^T (2) and R dh^T (2)
    assert bench.kernel_work("scalar")["bwd_local"][1] == unit * (4 + 5 + 4)
    # the seven-product graph adds 4 n^2 d_k + 4 n^3 FLOPs (3.15 M)
    extra = bench.kernel_work("scalar")["bwd_local_wy7"][1] - bench.kernel_work("scalar")["bwd_local"][1]
    assert extra == 3 * unit
    assert abs(extra - (4 * CH * CH * D + 4 * CH ** 3)) / extra < 0.002


def test_three_product_flops_are_the_pages_figure():
    with open(os.path.join(ROOT, "tests", "golden", "local_wy_flops.json")) as fh:
        gold = json.load(fh)
    a6 = 4 * bench.M                       # A^T Rbar, P R^T, P h^T
    assert round(a6 / 1e6, 2) == gold["rewy_millions"]


def _profile_algorithmic(path, stages):
    with open(path) as fh:
        text = fh.read()
    out = {}
    for st in stages:
        m = re.search(r"^\| %s \| \d+ \| \d+ \| (\d+) \|" % st, text, re.M)
        assert m, (path, st)
        out[st] = int(m.group(1))
    return out


@pytest.mark.parametrize("gate,path", [
    ("scalar", "profiles/gdn_bwd_R_1x8192x16_hbm_traffic.md"),
    ("vector", "profiles/kda_bwd_R_1x8192x16_stats_traffic.md"),
])
def test_profile_tables_use_the_same_figures(gate, path):
    stages = ["prep", "scan_pair", "bwd_local"]
    got = _profile_algorithmic(os.path.join(ROOT, path), stages)
    units = 1 * 8192 // CH * 16
    for st in stages:
        assert got[st] == bench.kernel_work(gate)[st][0] * units, st


def test_ablation_profile_uses_the_same_figures():
    with open(os.path.join(ROOT, "profiles", "gdn_bwd_R_1x8192x16_rewy_vs_wy7.md")) as fh:
        text = fh.read()
    w = bench.kernel_work("scalar")
    units = 8192 // CH * 16
    expect = {("bwd_local", "ReWY"): w["bwd_local"][0], ("bwd_local", "seven-product"): w["bwd_local_wy7"][0],
              ("scan_pair", "ReWY"): w["scan_pair"][0], ("prep", "ReWY"): w["prep"][0],
              # the seven-product backward's prep also writes A (64 x 64 bf16)
              ("prep", "seven-product"): w["prep"][0] + CH * CH * BF16}
    for (st, kind), per in expect.items():
        m = re.search(r"^\| %s \| %s \|(?: [0-9.]+ \|){4} ([0-9.]+) \|" % (st, kind), text, re.M)
        assert m, (st, kind)
        assert float(m.group(1)) == round(per * units / 1e6, 1), (st, kind)
