"""Pins of the chunkwise algebra: the chunk forms reproduce the token oracle
at every chunk size (including tails), the three-product ReWY backward equals
the seven-product expanded backward, the consumers (Gram elimination,
centred matrix intra) equal the dense route, and the counted FLOPs reproduce
the figures the pages print.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunk_forms as cf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _seq(gate, T, DK, DV, seed=0, strong=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, DK)) / np.sqrt(DK)
    k = rng.standard_normal((T, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, DV))
    gs = (T,) if gate == "scalar" else (T, DK)
    mean = 0.0 if strong else 3.0
    g = -np.logaddexp(0, -(rng.standard_normal(gs) + mean))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    beta[::3] = 0.0
    h0 = 0.1 * rng.standard_normal((DK, DV))
    dO = rng.standard_normal((T, DV))
    dht = 0.1 * rng.standard_normal((DK, DV))
    return q, k, v, g, beta, h0, dO, dht


def _token(q, k, v, g, beta, h0, dO, dht):
    B = lambda x: x[None, :, None]  # noqa: E731  (T,...) -> (1,T,1,...)
    o, ht = oracle.token_fwd(B(q), B(k), B(v), B(g), B(beta), h0[None, None])
    gr = oracle.token_bwd(B(q), B(k), B(v), B(g), B(beta), h0[None, None], B(dO), dht[None, None])
    gr = {n: (a[0, :, 0] if n != "dh0" else a[0, 0]) for n, a in gr.items()}
    return o[0, :, 0], ht[0, 0], gr


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("gate", ["scalar", "vector"])
@pytest.mark.parametrize("C", [1, 2, 4, 16, 64])
def test_chunk_forms_reproduce_token_oracle(gate, C):
    T = 150  # not a multiple of 4, 16 or 64: exercises the tail chunk
    q, k, v, g, beta, h0, dO, dht = _seq(gate, T, 8, 5, seed=C)
    o_t, ht_t, gr_t = _token(q, k, v, g, beta, h0, dO, dht)
    o_c, ht_c = cf.chunk_forward(q, k, v, g, beta, h0, C)
    assert _rel(o_c, o_t) < 1e-12
    assert _rel(ht_c, ht_t) < 1e-12
    gr_c = cf.chunk_backward(q, k, v, g, beta, h0, dO, dht, C, "rewy", "direct")
    for n in gr_t:
        assert _rel(gr_c[n], gr_t[n]) < 1e-10, n


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_three_product_equals_seven_product(gate):
    T, DK, DV = 192, 32, 16
    args = _seq(gate, T, DK, DV, seed=21)
    a = cf.chunk_backward(*args, 64, "rewy", "direct")
    b = cf.chunk_backward(*args, 64, "wy7", "direct")
    for n in a:
        assert _rel(a[n], b[n]) < 1e-10, n


def test_gram_elimination_equals_dense_route():
    args = _seq("scalar", 160, 16, 12, seed=31)
    a = cf.chunk_backward(*args, 64, "rewy", "direct")
    b = cf.chunk_backward(*args, 64, "rewy", "gram")
    for n in a:
        assert _rel(b[n], a[n]) < 1e-12, n


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_centred_matrix_intra_equals_dense_route(gate):
    args = _seq(gate, 160, 16, 12, seed=41, strong=True)
    a = cf.chunk_backward(*args, 64, "rewy", "direct")
    b = cf.chunk_backward(*args, 64, "rewy", "centred")
    for n in a:
        assert _rel(b[n], a[n]) < 1e-12, n


def test_centring_constant_cancels():
    """Any per-feature centre gives the same gradients (scaling invariance)."""
    args = _seq("vector", 128, 16, 8, seed=51)
    rng = np.random.default_rng(52)
    a = cf.chunk_backward(*args, 64, "rewy", "centred")
    b = cf.chunk_backward(*args, 64, "rewy", "centred",
                          centre=lambda G: rng.uniform(-3, 3, size=G.shape[1]))
    for n in a:
        assert _rel(b[n], a[n]) < 1e-12, n


def test_centring_bounds_the_factors():
    """With c = (max G + min G)/2 every centred factor is at most exp(range/2)."""
    rng = np.random.default_rng(61)
    g = -np.logaddexp(0, -(rng.standard_normal((64, 16)) + 3.0))
    G = np.cumsum(g, axis=0)
    c = 0.5 * (G.max(0) + G.min(0))
    half = 0.5 * (G.max(0) - G.min(0))
    assert np.all(np.abs(G - c) <= half + 1e-15)


def test_local_wy_flops_match_the_pages():
    gold = json.load(open(os.path.join(GOLDEN, "local_wy_flops.json")))
    n, dk, dv = gold["n"], gold["dk"], gold["dv"]
    f7, c7 = cf.local_wy_flops(n, dk, dv, "wy7")
    f3, c3 = cf.local_wy_flops(n, dk, dv, "rewy")
    assert (c7, c3) == (gold["wy7_products"], gold["rewy_products"])
    assert round(f7 / 1e6, 2) == gold["wy7_millions"]
    assert round(f3 / 1e6, 2) == gold["rewy_millions"]
    assert round(100 * (f7 - f3) / f7, 1) == gold["removed_percent"]


@pytest.mark.parametrize("n,dk,dv", [(64, 128, 128), (16, 8, 4), (32, 64, 96), (8, 3, 7)])
def test_removed_flops_identity(n, dk, dv):
    """dF = 4 n^2 d_k + 4 n^3, independent of d_v (onedev.kr summary)."""
    f7, _ = cf.local_wy_flops(n, dk, dv, "wy7")
    f3, _ = cf.local_wy_flops(n, dk, dv, "rewy")
    assert f7 - f3 == 4 * n * n * dk + 4 * n ** 3


def _strong(gate, T, DK, DV, seed, lo=-5.0):
    """Inputs whose log decays are drawn uniformly from [lo, 0] (strong decay:
    a 64-token chunk spans a log-decay range of about 64 |lo| / 2)."""
    q, k, v, g, beta, h0, dO, dht = _seq(gate, T, DK, DV, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    g = rng.uniform(lo, 0.0, size=g.shape)
    return q, k, v, g, beta, h0, dO, dht


@pytest.mark.parametrize("gate", ["scalar", "vector"])
@pytest.mark.parametrize("window", [32, 16, 7])
def test_windowed_matrix_intra_equals_dense_route(gate, window):
    args = _seq(gate, 150, 16, 12, seed=71, strong=True)  # 150: a ragged last chunk
    a = cf.chunk_backward(*args, 64, "rewy", "direct")
    b = cf.chunk_backward(*args, 64, "rewy", "windowed", window=window)
    for n in a:
        assert _rel(b[n], a[n]) < 1e-12, n


@pytest.mark.parametrize("producer", ["rewy", "wy7"])
@pytest.mark.parametrize("lo", [-5.0, -10.0])
def test_windowed_reproduces_token_oracle_under_strong_decay(producer, lo):
    """|g| up to 5 (10) per token: a chunk's range reaches about 160 (320),
    a 16-token window about 40 (80). The windowed chunk form, in fp64,
    equals the token recurrence."""
    q, k, v, g, beta, h0, dO, dht = _strong("vector", 150, 8, 5, seed=81, lo=lo)
    o_t, ht_t, gr_t = _token(q, k, v, g, beta, h0, dO, dht)
    gr_c = cf.chunk_backward(q, k, v, g, beta, h0, dO, dht, 64, producer, "windowed")
    for n in gr_t:
        assert _rel(gr_c[n], gr_t[n]) < 1e-10, n


def test_windowed_factors_stay_within_fp32_range():
    """Under per-token decays down to exp(-10), the window-centred factors of
    16-token windows stay within exp(+-80), while centring per 32-token
    window needs factors beyond exp(88), past the largest fp32. Every other
    exponent is at most 0 (it can only underflow, towards a product that is
    that small): the boundary-pivot factors, G[16 m - 1] against earlier
    windows and G[16 m + 16] against later ones, and the per-key scales
    exp(G[16 m - 1] - c_w), exp(c_w - G[16 m + 16]) that turn a
    window-centred operand into a boundary-pivot one."""
    rng = np.random.default_rng(91)
    worst16, worst32 = 0.0, 0.0
    for _ in range(50):
        g = rng.uniform(-10.0, 0.0, size=(64, 128))
        G = np.cumsum(g, axis=0)
        c = [0.5 * (G[16 * m:16 * m + 16].max(0) + G[16 * m:16 * m + 16].min(0)) for m in range(4)]
        for m in range(4):
            W = G[16 * m:16 * m + 16]
            worst16 = max(worst16, np.abs(W - c[m]).max())
            if m >= 1:  # rows of window m against earlier columns
                p = G[16 * m - 1]
                assert np.all(W - p <= 0) and np.all(p - G[:16 * m] <= 0)
                for w in range(m):
                    assert np.all(p - c[w] <= 0)
            if m <= 2:  # rows of window m against later columns
                p = G[16 * m + 16]
                assert np.all(p - W <= 0) and np.all(G[16 * m + 16:] - p <= 0)
                for w in range(m + 1, 4):
                    assert np.all(c[w] - p <= 0)
        for a0 in (0, 32):
            W = G[a0:a0 + 32]
            worst32 = max(worst32, np.abs(W - 0.5 * (W.max(0) + W.min(0))).max())
    assert worst16 <= 80.0
    assert worst32 > 88.0


@pytest.mark.parametrize("n", [64, 45])
@pytest.mark.parametrize("incl", [True, False])
def test_pivoted_lower_equals_pairwise_definition(n, incl):
    """The tile-pivoted product equals its definition entry by entry,
    sum_f X_if Y_jf exp(G_if - G_jf), each exponent formed per pair, under
    decays strong enough that exp(-G) alone would leave fp32."""
    rng = np.random.default_rng(100 + n)
    X = rng.standard_normal((n, 12))
    Y = rng.standard_normal((n, 12))
    G = np.cumsum(rng.uniform(-5.0, 0.0, size=(n, 12)), axis=0)
    ref = np.zeros((n, n))
    for i in range(n):
        for j in range(i + 1 if incl else i):
            ref[i, j] = np.sum(X[i] * Y[j] * np.exp(G[i] - G[j]))
    got = cf.pivoted_lower(X, Y, G, incl)
    assert np.max(np.abs(got - ref)) <= 1e-12 * max(np.max(np.abs(ref)), 1.0)


# ------------------------------------------------------------------ GDN2

def _gdn2_seq(T, DK, DV, seed=0, mean=3.0):
    q, k, v, g, beta, h0, dO, dht = _seq("vector", T, DK, DV, seed=seed)
    rng = np.random.default_rng(seed + 100)
    g = -np.logaddexp(0, -(rng.standard_normal((T, DK)) + mean))
    ers = 1 / (1 + np.exp(-rng.standard_normal((T, DK))))
    wrt = 1 / (1 + np.exp(-rng.standard_normal((T, DV))))
    ers[::5] = 0.0
    wrt[1::7] = 0.0
    return q, k, v, g, ers, wrt, h0, dO, dht


def _gdn2_token(q, k, v, g, ers, wrt, h0, dO, dht):
    B = lambda x: x[None, :, None]  # noqa: E731
    o, ht = oracle.gdn2_fwd(B(q), B(k), B(v), B(g), B(ers), B(wrt), h0[None, None])
    gr = oracle.gdn2_bwd(B(q), B(k), B(v), B(g), B(ers), B(wrt), h0[None, None], B(dO),
                         dht[None, None])
    gr = {n: (a[0, :, 0] if n != "dh0" else a[0, 0]) for n, a in gr.items()}
    return o[0, :, 0], ht[0, 0], gr


@pytest.mark.parametrize("C", [1, 4, 16, 64])
@pytest.mark.parametrize("producer, consumer", [("rewy", "direct"), ("wy7", "direct"),
                                                ("rewy", "windowed")])
def test_gdn2_chunk_forms_reproduce_token_oracle(C, producer, consumer):
    """GDN2 chunk forms (E = ers o gam o K, Z = wrt o V) equal the GDN2 token
    oracle at every chunk size with a tail, for both producers and for the
    windowed matrix-intra consumer the device kernels use."""
    T = 150
    x = _gdn2_seq(T, 8, 5, seed=C)
    q, k, v, g, ers, wrt, h0, dO, dht = x
    o_t, ht_t, gr_t = _gdn2_token(*x)
    o_c, ht_c = cf.chunk_forward(q, k, v, g, None, h0, C, ers=ers, wrt=wrt)
    assert _rel(o_c, o_t) < 1e-12
    assert _rel(ht_c, ht_t) < 1e-12
    gr_c = cf.chunk_backward(q, k, v, g, None, h0, dO, dht, C, producer, consumer,
                             ers=ers, wrt=wrt)
    assert set(gr_c) == set(gr_t)
    for n in gr_t:
        assert _rel(gr_c[n], gr_t[n]) < 1e-10, n


def test_gdn2_windowed_under_strong_decay():
    """Per-token decays around e^-4 (chunk range ~256): the windowed GDN2
    consumer stays finite and equals the token oracle."""
    x = _gdn2_seq(130, 8, 5, seed=3, mean=-4.0)
    q, k, v, g, ers, wrt, h0, dO, dht = x
    _, _, gr_t = _gdn2_token(*x)
    gr_c = cf.chunk_backward(q, k, v, g, None, h0, dO, dht, 64, "rewy", "windowed",
                             ers=ers, wrt=wrt)
    for n in gr_t:
        assert np.all(np.isfinite(gr_c[n])), n
        assert _rel(gr_c[n], gr_t[n]) < 1e-9, n
