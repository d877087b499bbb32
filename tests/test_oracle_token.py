"""Pins of the token-by-token fp64 oracle against things other than itself:
complex-step derivatives of its own forward (an independent arithmetic route
to every gradient), central differences, and closed forms of the recurrence.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tiny(gate, seed=1, B=1, T=7, H=2, DK=3, DV=2, zero_beta=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, DK)) * 0.7
    k = rng.standard_normal((B, T, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    gs = (B, T, H) if gate == "scalar" else (B, T, H, DK)
    g = -np.logaddexp(0, -(rng.standard_normal(gs) + 1.0))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    if zero_beta:
        beta[0, 2, 0] = 0.0          # exactly zero weight
        beta[0, 4, 1] = 1e-9         # tiny weight
    h0 = 0.3 * rng.standard_normal((B, H, DK, DV))
    dO = rng.standard_normal((B, T, H, DV))
    dht = 0.5 * rng.standard_normal((B, H, DK, DV))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0, dO=dO, dht=dht)


def _objective(x, complex_=False):
    fwd = oracle.token_fwd_complex if complex_ else oracle.token_fwd
    o, ht = fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    return np.sum(o * x["dO"]) + np.sum(ht * x["dht"])


NAMES = ["q", "k", "v", "g", "beta", "h0"]
GRAD = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_backward_matches_complex_step_elementwise(gate):
    """Every gradient entry equals Im f(x + i h e_idx) / h of the forward."""
    x = _tiny(gate)
    grads = oracle.token_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["dO"], x["dht"],
                             threads=3)
    hstep = 1e-30
    for name in NAMES:
        ref = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xc = {kk: np.asarray(vv, dtype=np.complex128) for kk, vv in x.items()}
            xc[name] = xc[name].copy()
            xc[name][idx] += 1j * hstep
            ref[idx] = np.imag(_objective(xc, complex_=True)) / hstep
        got = grads[GRAD[name]]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_backward_matches_central_differences(gate):
    """Directional derivatives along random directions, central differences."""
    x = _tiny(gate, seed=5, T=9)
    grads = oracle.token_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["dO"], x["dht"])
    rng = np.random.default_rng(11)
    eps = 1e-6
    for name in NAMES:
        d = rng.standard_normal(x[name].shape)
        xp = dict(x)
        xm = dict(x)
        xp[name] = x[name] + eps * d
        xm[name] = x[name] - eps * d
        fd = (_objective(xp) - _objective(xm)) / (2 * eps)
        an = np.sum(grads[GRAD[name]] * d)
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_complex_forward_equals_real_forward():
    x = _tiny("vector", seed=2)
    o, ht = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    oc, htc = oracle.token_fwd_complex(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    np.testing.assert_array_equal(o, oc.real)
    np.testing.assert_array_equal(ht, htc.real)


@pytest.mark.parametrize("gate", ["scalar", "vector"])
def test_zero_beta_is_pure_decay(gate):
    """beta = 0: no writes, the state only decays, o_t = h0^T (prod a) q_t."""
    x = _tiny(gate, seed=3, T=6)
    beta = np.zeros_like(x["beta"])
    o, ht = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], beta, x["h0"])
    B, T, H, DK = x["q"].shape
    G = np.cumsum(x["g"], axis=1)
    if gate == "scalar":
        G = np.repeat(G[..., None], DK, axis=-1)
    dec = np.exp(G)  # [B,T,H,DK]
    ref_o = np.einsum("bthk,bhkv->bthv", dec * x["q"], x["h0"])
    ref_ht = dec[:, -1][..., None] * x["h0"]
    np.testing.assert_allclose(o, ref_o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ht, ref_ht, rtol=1e-13, atol=1e-14)


def test_overwrite_memory_with_one_hot_keys():
    """g = 0, beta = 1, one-hot keys: each write replaces the value stored
    under that key (the textbook delta-rule overwrite memory)."""
    B, T, H, DK, DV = 1, 11, 1, 4, 3
    rng = np.random.default_rng(4)
    keys = rng.integers(0, DK, size=T)
    k = np.zeros((B, T, H, DK))
    k[0, np.arange(T), 0, keys] = 1.0
    q = rng.standard_normal((B, T, H, DK))
    v = rng.standard_normal((B, T, H, DV))
    g = np.zeros((B, T, H))
    beta = np.ones((B, T, H))
    h0 = rng.standard_normal((B, H, DK, DV))
    o, ht = oracle.token_fwd(q, k, v, g, beta, h0)
    mem = h0[0, 0].copy()  # [DK, DV]: value stored under each key
    for t in range(T):
        mem[keys[t]] = v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], q[0, t, 0] @ mem, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ht[0, 0], mem, rtol=1e-13, atol=1e-13)


def test_unit_weight_write_is_recalled_exactly():
    """beta = 1 and |k| = 1: right after the write, X_t k_t = v_t, so a query
    equal to the key reads back exactly the written value (any decay)."""
    x = _tiny("vector", seed=6, T=8, zero_beta=False)
    beta = np.ones_like(x["beta"])
    q = x["k"].copy()
    o, _ = oracle.token_fwd(q, x["k"], x["v"], x["g"], beta, x["h0"])
    np.testing.assert_allclose(o, x["v"], rtol=1e-12, atol=1e-12)


def test_linear_in_values_and_initial_state():
    x = _tiny("scalar", seed=7)
    rng = np.random.default_rng(8)
    v2 = rng.standard_normal(x["v"].shape)
    h2 = rng.standard_normal(x["h0"].shape)
    a = 0.37
    o1, t1 = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o2, t2 = oracle.token_fwd(x["q"], x["k"], v2, x["g"], x["beta"], h2)
    o3, t3 = oracle.token_fwd(x["q"], x["k"], a * x["v"] + v2, x["g"], x["beta"], a * x["h0"] + h2)
    np.testing.assert_allclose(o3, a * o1 + o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(t3, a * t1 + t2, rtol=1e-12, atol=1e-12)


def test_vector_gate_broadcast_equals_scalar_gate():
    """A per-channel gate that is the same on every channel is the scalar
    gate; its gradient summed over channels is the scalar gradient."""
    xs = _tiny("scalar", seed=9)
    DK = xs["q"].shape[-1]
    gv = np.repeat(xs["g"][..., None], DK, axis=-1)
    os_, hs = oracle.token_fwd(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"])
    ov, hv = oracle.token_fwd(xs["q"], xs["k"], xs["v"], gv, xs["beta"], xs["h0"])
    np.testing.assert_allclose(ov, os_, rtol=1e-13, atol=1e-14)
    gs = oracle.token_bwd(xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["h0"], xs["dO"], xs["dht"])
    gvv = oracle.token_bwd(xs["q"], xs["k"], xs["v"], gv, xs["beta"], xs["h0"], xs["dO"], xs["dht"])
    np.testing.assert_allclose(gvv["dg"].sum(-1), gs["dg"], rtol=1e-11, atol=1e-13)
    for n in ("dq", "dk", "dv", "dbeta", "dh0"):
        np.testing.assert_allclose(gvv[n], gs[n], rtol=1e-11, atol=1e-13)


def test_result_independent_of_thread_count():
    x = _tiny("vector", seed=10, T=150, H=3, DK=6, DV=9)
    a = oracle.token_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["dO"], x["dht"], threads=1)
    b = oracle.token_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["dO"], x["dht"], threads=7)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n], err_msg=n)
    o1, _ = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], threads=1)
    o2, _ = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], threads=5)
    np.testing.assert_array_equal(o1, o2)


def test_empty_sequence():
    x = _tiny("scalar", T=0, zero_beta=False)
    o, ht = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    assert o.shape[1] == 0
    np.testing.assert_array_equal(ht, x["h0"])
    gr = oracle.token_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], x["dO"], x["dht"])
    np.testing.assert_array_equal(gr["dh0"], x["dht"])
