"""Pins of the GDN2 token oracle (per-key-channel decay with independent
erase and write gates, ReWY paper Table 1; Sec. 3.1 keeps their gradients
separate) against things other than itself:

- complex-step derivatives of its own forward, entry by entry, for all seven
  gradients (an independent arithmetic route to each of them);
- the exact reduction to the KDA oracle (itself pinned in
  test_oracle_token.py) when both gates equal beta in every channel: same
  outputs and state, same gradients, and dbeta = sum of the erase and write
  gradients over their channels (App. E.1: a shared parameter's adjoint is
  the sum over the paths that use it);
- one-hot keys without decay, where each key slot keeps (1 - erase) of its
  content and receives the write-gated value: which side each gate scales;
- no erase at all, where the recurrence is gated linear attention with a
  closed form written as explicit sums over tokens.
"""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _tiny(seed=1, B=1, T=7, H=2, DK=3, DV=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, DK)) * 0.7
    k = rng.standard_normal((B, T, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, DV))
    g = -np.logaddexp(0, -(rng.standard_normal((B, T, H, DK)) + 1.0))
    ers = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, DK))))
    wrt = 1 / (1 + np.exp(-rng.standard_normal((B, T, H, DV))))
    ers[0, 2, 0, 1] = 0.0           # an erase channel switched off
    wrt[0, 4, H - 1, 0] = 0.0       # a write channel switched off
    h0 = 0.3 * rng.standard_normal((B, H, DK, DV))
    dO = rng.standard_normal((B, T, H, DV))
    dht = 0.5 * rng.standard_normal((B, H, DK, DV))
    return dict(q=q, k=k, v=v, g=g, ers=ers, wrt=wrt, h0=h0, dO=dO, dht=dht)


def _objective(x, complex_=False):
    fwd = oracle.gdn2_fwd_complex if complex_ else oracle.gdn2_fwd
    o, ht = fwd(x["q"], x["k"], x["v"], x["g"], x["ers"], x["wrt"], x["h0"])
    return np.sum(o * x["dO"]) + np.sum(ht * x["dht"])


NAMES = ["q", "k", "v", "g", "ers", "wrt", "h0"]
GRAD = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "ers": "ders", "wrt": "dwrt", "h0": "dh0"}


def _bwd(x, threads=None):
    return oracle.gdn2_bwd(x["q"], x["k"], x["v"], x["g"], x["ers"], x["wrt"], x["h0"], x["dO"],
                           x["dht"], threads=threads)


def test_gdn2_backward_matches_complex_step_elementwise():
    x = _tiny()
    grads = _bwd(x, threads=3)
    hstep = 1e-30
    for name in NAMES:
        ref = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xc = {kk: np.asarray(vv, dtype=np.complex128) for kk, vv in x.items()}
            xc[name] = xc[name].copy()
            xc[name][idx] += 1j * hstep
            ref[idx] = np.imag(_objective(xc, complex_=True)) / hstep
        np.testing.assert_allclose(grads[GRAD[name]], ref, rtol=1e-12, atol=1e-13, err_msg=name)


def test_gdn2_complex_forward_equals_real_forward():
    x = _tiny(seed=2)
    o, ht = oracle.gdn2_fwd(x["q"], x["k"], x["v"], x["g"], x["ers"], x["wrt"], x["h0"])
    oc, htc = oracle.gdn2_fwd_complex(x["q"], x["k"], x["v"], x["g"], x["ers"], x["wrt"], x["h0"])
    np.testing.assert_array_equal(o, oc.real)
    np.testing.assert_array_equal(ht, htc.real)


@pytest.mark.parametrize("T", [7, 130])
def test_gdn2_with_shared_gates_is_kda(T):
    """erase = write = beta in every channel gives the KDA recurrence; the
    beta gradient is the sum of the two gate gradients over their channels."""
    x = _tiny(seed=4, T=T, H=3, DK=4, DV=3)
    rng = np.random.default_rng(9)
    beta = 1 / (1 + np.exp(-rng.standard_normal(x["q"].shape[:3])))
    beta[0, 1, 0] = 0.0
    ers = np.repeat(beta[..., None], x["q"].shape[-1], axis=-1)
    wrt = np.repeat(beta[..., None], x["v"].shape[-1], axis=-1)
    o1, h1 = oracle.token_fwd(x["q"], x["k"], x["v"], x["g"], beta, x["h0"])
    o2, h2 = oracle.gdn2_fwd(x["q"], x["k"], x["v"], x["g"], ers, wrt, x["h0"])
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h2, h1, rtol=1e-12, atol=1e-13)
    g1 = oracle.token_bwd(x["q"], x["k"], x["v"], x["g"], beta, x["h0"], x["dO"], x["dht"])
    g2 = oracle.gdn2_bwd(x["q"], x["k"], x["v"], x["g"], ers, wrt, x["h0"], x["dO"], x["dht"])
    for n in ("dq", "dk", "dv", "dg", "dh0"):
        np.testing.assert_allclose(g2[n], g1[n], rtol=1e-11, atol=1e-12, err_msg=n)
    np.testing.assert_allclose(g2["ders"].sum(-1) + g2["dwrt"].sum(-1), g1["dbeta"],
                               rtol=1e-11, atol=1e-12)


def test_gdn2_one_hot_keys_erase_and_write_per_slot():
    """No decay, k_t = e_{i_t}: slot i_t (a key row of the key-major state)
    becomes (1 - ers_t[i_t]) * slot + wrt_t o v_t; the other slots are kept.
    This fixes that the erase gate scales the key side and the write gate
    the value side."""
    rng = np.random.default_rng(12)
    B, T, H, DK, DV = 1, 9, 1, 4, 3
    slots = rng.integers(0, DK, size=T)
    k = np.zeros((B, T, H, DK))
    k[0, np.arange(T), 0, slots] = 1.0
    q = rng.standard_normal((B, T, H, DK))
    v = rng.standard_normal((B, T, H, DV))
    g = np.zeros((B, T, H, DK))
    ers = rng.uniform(0, 1, (B, T, H, DK))
    wrt = rng.uniform(0, 1, (B, T, H, DV))
    h0 = rng.standard_normal((B, H, DK, DV))
    o, ht = oracle.gdn2_fwd(q, k, v, g, ers, wrt, h0)
    S = h0[0, 0].copy()
    for t in range(T):
        i = slots[t]
        S[i] = (1 - ers[0, t, 0, i]) * S[i] + wrt[0, t, 0] * v[0, t, 0]
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[0, t, 0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-13, atol=1e-14)


def test_gdn2_without_erase_is_gated_linear_attention():
    """ers = 0: S_t = Diag(a_t) S_{t-1} + k_t (wrt_t o v_t)^T, so
    o_t = sum_{s <= t} <q_t, prod_{s < u <= t} a_u o k_s> (wrt_s o v_s)
          + (prod_{u <= t} a_u o q_t)^T h0, written out term by term."""
    x = _tiny(seed=6, T=8, H=1, DK=3, DV=2)
    ers = np.zeros_like(x["ers"])
    o, ht = oracle.gdn2_fwd(x["q"], x["k"], x["v"], x["g"], ers, x["wrt"], x["h0"])
    q, k, v, g, wrt, h0 = (x[n][0, :, 0] if n != "h0" else x[n][0, 0]
                           for n in ("q", "k", "v", "g", "wrt", "h0"))
    T = q.shape[0]
    for t in range(T):
        ref = (np.exp(g[:t + 1].sum(0)) * q[t]) @ h0
        for s in range(t + 1):
            dec = np.exp(g[s + 1:t + 1].sum(0))
            ref = ref + np.dot(q[t], dec * k[s]) * (wrt[s] * v[s])
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=1e-12, atol=1e-13)


def test_gdn2_result_independent_of_thread_count():
    x = _tiny(seed=8, T=40, H=3, DK=5, DV=6)
    a, b = _bwd(x, threads=1), _bwd(x, threads=7)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
