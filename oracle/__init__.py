"""fp64 CPU oracle for chunkwise gated delta-rule attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the GPU library (``delta_rule_linear_gdr_amd``) and never imports it;
both sides only share the seeded input generator, which holds none of the
method's arithmetic.

Contents
  token_fwd / token_bwd   ctypes wrappers of ``gdr_oracle.c``: the plain
                          token-by-token recurrence (ReWY paper, Sec. 2.2,
                          Table 1) and its hand-derived reverse mode.
  gdn2_fwd / gdn2_bwd     the same for GDN2 (paper Table 1: per-key-channel
                          decay, independent erase gate per key channel and
                          write gate per value channel, in place of beta),
                          and gdn2_fwd_complex.
  token_fwd_complex       the same recurrence in complex arithmetic, for
                          complex-step derivative checks (paper Sec. 4.5 and
                          App. G.3 name CPU FP64 and complex-step checks).
  chunk_forms             numpy fp64 chunkwise forms (WY forward, the
                          three-product ReWY backward, the seven-product
                          expanded WY backward, Gram elimination, centred
                          matrix intra) with a FLOP counter; they pin the
                          token oracle and the algebra.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_HDR = os.path.join(_HERE, "token_fwd_body.h")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gdr_oracle.c with gcc into oracle/libgdr_oracle.so."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            os.path.getmtime(_SRC), os.path.getmtime(_HDR)):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.gdr_oracle_fwd.argtypes = [i64] * 5 + [i32] + [p] * 8 + [i32]
    lib.gdr_oracle_fwd.restype = i32
    lib.gdr_oracle_fwd_complex.argtypes = [i64] * 5 + [i32] + [p] * 8
    lib.gdr_oracle_fwd_complex.restype = i32
    lib.gdr_oracle_bwd.argtypes = [i64] * 5 + [i32] + [p] * 14 + [i32]
    lib.gdr_oracle_bwd.restype = i32
    lib.gdr_oracle_gdn2_fwd.argtypes = [i64] * 5 + [p] * 9 + [i32]
    lib.gdr_oracle_gdn2_fwd.restype = i32
    lib.gdr_oracle_gdn2_fwd_complex.argtypes = [i64] * 5 + [p] * 9
    lib.gdr_oracle_gdn2_fwd_complex.restype = i32
    lib.gdr_oracle_gdn2_bwd.argtypes = [i64] * 5 + [p] * 16 + [i32]
    lib.gdr_oracle_gdn2_bwd.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _arr(x, dtype=np.float64):
    return np.ascontiguousarray(x, dtype=dtype)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _dims(q, v, g):
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    vec = 1 if g.ndim == 4 else 0
    return B, T, H, DK, DV, vec


def token_fwd(q, k, v, g, beta, h0=None, threads: int | None = None):
    """Forward recurrence in fp64. Returns (o [B,T,H,DV], ht [B,H,DK,DV])."""
    lib = _load()
    q, k, v, g, beta = (_arr(x) for x in (q, k, v, g, beta))
    h0 = None if h0 is None else _arr(h0)
    B, T, H, DK, DV, vec = _dims(q, v, g)
    o = np.zeros((B, T, H, DV))
    ht = np.zeros((B, H, DK, DV))
    rc = lib.gdr_oracle_fwd(B, T, H, DK, DV, vec, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                            _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
                            threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_fwd failed ({rc})")
    return o, ht


def token_fwd_complex(q, k, v, g, beta, h0=None):
    """Forward recurrence in complex128 (single thread), for complex-step checks."""
    lib = _load()
    c = np.complex128
    q, k, v, g, beta = (_arr(x, c) for x in (q, k, v, g, beta))
    h0 = None if h0 is None else _arr(h0, c)
    B, T, H, DK, DV, vec = _dims(q, v, g)
    o = np.zeros((B, T, H, DV), c)
    ht = np.zeros((B, H, DK, DV), c)
    rc = lib.gdr_oracle_fwd_complex(B, T, H, DK, DV, vec, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht))
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_fwd_complex failed ({rc})")
    return o, ht


def token_bwd(q, k, v, g, beta, h0, dO, dht=None, threads: int | None = None):
    """Exact gradients of <o, dO> + <ht, dht>. Returns dict dq, dk, dv, dg, dbeta, dh0."""
    lib = _load()
    q, k, v, g, beta, dO = (_arr(x) for x in (q, k, v, g, beta, dO))
    h0 = None if h0 is None else _arr(h0)
    dht = None if dht is None else _arr(dht)
    B, T, H, DK, DV, vec = _dims(q, v, g)
    out = {
        "dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
        "dg": np.zeros_like(g), "dbeta": np.zeros_like(beta),
        "dh0": np.zeros((B, H, DK, DV)),
    }
    rc = lib.gdr_oracle_bwd(B, T, H, DK, DV, vec, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                            _ptr(beta), _ptr(h0), _ptr(dO), _ptr(dht), _ptr(out["dq"]),
                            _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                            _ptr(out["dbeta"]), _ptr(out["dh0"]),
                            threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_bwd failed ({rc})")
    return out


def gdn2_fwd(q, k, v, g, ers, wrt, h0=None, threads: int | None = None):
    """GDN2 forward in fp64: g, ers [B,T,H,DK], wrt [B,T,H,DV]. Returns (o, ht)."""
    lib = _load()
    q, k, v, g, ers, wrt = (_arr(x) for x in (q, k, v, g, ers, wrt))
    h0 = None if h0 is None else _arr(h0)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    assert g.shape == (B, T, H, DK) and ers.shape == (B, T, H, DK) and wrt.shape == (B, T, H, DV)
    o = np.zeros((B, T, H, DV))
    ht = np.zeros((B, H, DK, DV))
    rc = lib.gdr_oracle_gdn2_fwd(B, T, H, DK, DV, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(ers),
                                 _ptr(wrt), _ptr(h0), _ptr(o), _ptr(ht),
                                 threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_gdn2_fwd failed ({rc})")
    return o, ht


def gdn2_fwd_complex(q, k, v, g, ers, wrt, h0=None):
    """GDN2 forward in complex128 (single thread), for complex-step checks."""
    lib = _load()
    c = np.complex128
    q, k, v, g, ers, wrt = (_arr(x, c) for x in (q, k, v, g, ers, wrt))
    h0 = None if h0 is None else _arr(h0, c)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    o = np.zeros((B, T, H, DV), c)
    ht = np.zeros((B, H, DK, DV), c)
    rc = lib.gdr_oracle_gdn2_fwd_complex(B, T, H, DK, DV, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                         _ptr(ers), _ptr(wrt), _ptr(h0), _ptr(o), _ptr(ht))
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_gdn2_fwd_complex failed ({rc})")
    return o, ht


def gdn2_bwd(q, k, v, g, ers, wrt, h0, dO, dht=None, threads: int | None = None):
    """Exact GDN2 gradients of <o, dO> + <ht, dht>. Returns dict dq, dk, dv,
    dg, ders, dwrt, dh0."""
    lib = _load()
    q, k, v, g, ers, wrt, dO = (_arr(x) for x in (q, k, v, g, ers, wrt, dO))
    h0 = None if h0 is None else _arr(h0)
    dht = None if dht is None else _arr(dht)
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    out = {"dq": np.zeros_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "dg": np.zeros_like(g), "ders": np.zeros_like(ers), "dwrt": np.zeros_like(wrt),
           "dh0": np.zeros((B, H, DK, DV))}
    rc = lib.gdr_oracle_gdn2_bwd(B, T, H, DK, DV, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(ers),
                                 _ptr(wrt), _ptr(h0), _ptr(dO), _ptr(dht), _ptr(out["dq"]),
                                 _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                 _ptr(out["ders"]), _ptr(out["dwrt"]), _ptr(out["dh0"]),
                                 threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_gdn2_bwd failed ({rc})")
    return out
