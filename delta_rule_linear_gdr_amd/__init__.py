"""MI355X (gfx950) chunkwise gated delta-rule attention with the ReWY backward.

Thin Python binding over ``libgdr.so`` (C ABI in include/gdr.h): the
functions below only marshal torch device tensors into pointers and sizes and
pick up torch's current HIP stream. Every step of the computation runs in the
library's HIP kernels; there is no CPU or PyTorch fallback, and a missing or
unbuilt library raises.

    o, ht, saved = gdr_fwd(q, k, v, g, beta, h0, policy="recompute")
    grads = gdr_bwd(q, k, v, g, beta, h0, dO, dht, saved=saved, policy="recompute")
    grads = gdr_bwd_wy7(...)          # seven-product producer (ablation)
    o, ht, saved = gdr_fwd_gdn2(q, k, v, g, erase, write, h0)      # GDN2
    grads = gdr_bwd_gdn2(q, k, v, g, erase, write, h0, dO, dht, saved=saved)
    o, ht = chunk_gated_delta_rule(q, k, v, g, beta, h0)   # autograd-aware

Shapes: q, k [B,T,H,DK]; v, dO [B,T,H,DV]; g [B,T,H] (GDN, scalar gate),
[B,T,H,DK] (KDA, per-channel gate), fp32, or None (DeltaNet: no decay, and
no dg); beta [B,T,H]; h0, dht [B,H,DK,DV] fp32 (key-major) or None.
DK <= 128 and DV <= 1024 (widths below 128 through zero-padded copies, value
widths above 128 as 128-wide value blocks). q, k, v, beta, dO share one
dtype, bfloat16 or float32. Any T (a ragged last chunk is handled).

Packed variable-length batches: pass ``cu_seqlens`` (int64 device tensor of
n_seq + 1 token offsets) with batch size 1; the states h0, ht, dht, dh0 are
then [n_seq,H,DK,DV].
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["gdr_fwd", "gdr_bwd", "gdr_bwd_wy7", "gdr_fwd_gdn2", "gdr_bwd_gdn2",
           "chunk_gated_delta_rule", "chunk_gdn2", "workspace_size",
           "library_path", "load",
           "profile_begin", "profile_end", "set_local_form", "set_walk_levels", "gate_status",
           "GdrError",
           "RECOMPUTE", "FULL_SAVE"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdr.so")
_lib = None

RECOMPUTE, FULL_SAVE = 0, 1
GATE_SCALAR, GATE_VECTOR, GATE_NONE, GATE_GDN2 = 0, 1, 2, 3
DT_BF16, DT_F32 = 0, 1
STATUS = {0: "GDR_OK", -1: "GDR_ERR_INVALID", -2: "GDR_ERR_UNSUPPORTED",
          -3: "GDR_ERR_WORKSPACE", -4: "GDR_ERR_HIP"}
EXPORTS = ("gdr_workspace_size", "gdr_fwd", "gdr_bwd", "gdr_bwd_wy7",
           "gdr_fwd_gdn2", "gdr_bwd_gdn2", "gdr_fwd_gdn2_varlen", "gdr_bwd_gdn2_varlen",
           "gdr_bwd_noalloc", "gdr_workspace_size_varlen", "gdr_fwd_varlen", "gdr_bwd_varlen",
           "gdr_profile_begin", "gdr_profile_end", "gdr_set_local_form", "gdr_set_walk_levels",
           "gdr_gate_status", "gdr_status_string", "gdr_last_error", "gdr_version")


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class StageTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("DK", ctypes.c_int64), ("DV", ctypes.c_int64), ("C", ctypes.c_int64),
                ("gate", ctypes.c_int32), ("dtype", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dp = ctypes.POINTER(Desc)
    lib.gdr_workspace_size.argtypes = [dp, i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.gdr_workspace_size.restype = i32
    lib.gdr_fwd.argtypes = [dp, i32] + [p] * 10 + [sz, p]
    lib.gdr_fwd.restype = i32
    for name in ("gdr_bwd", "gdr_bwd_wy7"):
        fn = getattr(lib, name)
        fn.argtypes = [dp, i32] + [p] * 16 + [sz, p]
        fn.restype = i32
    lib.gdr_fwd_gdn2.argtypes = [dp, i32] + [p] * 11 + [sz, p]
    lib.gdr_fwd_gdn2.restype = i32
    lib.gdr_bwd_gdn2.argtypes = [dp, i32] + [p] * 18 + [sz, p]
    lib.gdr_bwd_gdn2.restype = i32
    lib.gdr_fwd_gdn2_varlen.argtypes = [dp, i32, p, ctypes.c_int64] + [p] * 11 + [sz, p]
    lib.gdr_fwd_gdn2_varlen.restype = i32
    lib.gdr_bwd_gdn2_varlen.argtypes = [dp, i32, p, ctypes.c_int64] + [p] * 18 + [sz, p]
    lib.gdr_bwd_gdn2_varlen.restype = i32
    lib.gdr_bwd_noalloc.argtypes = [dp, i32] + [p] * 16
    lib.gdr_bwd_noalloc.restype = i32
    i64 = ctypes.c_int64
    lib.gdr_workspace_size_varlen.argtypes = [dp, i64, i32, ctypes.POINTER(sz),
                                              ctypes.POINTER(sz)]
    lib.gdr_workspace_size_varlen.restype = i32
    lib.gdr_fwd_varlen.argtypes = [dp, i32, p, i64] + [p] * 10 + [sz, p]
    lib.gdr_fwd_varlen.restype = i32
    lib.gdr_bwd_varlen.argtypes = [dp, i32, p, i64] + [p] * 16 + [sz, p]
    lib.gdr_bwd_varlen.restype = i32
    lib.gdr_profile_begin.argtypes = [i32]
    lib.gdr_profile_begin.restype = i32
    lib.gdr_profile_end.argtypes = [ctypes.POINTER(StageTime), i32, ctypes.POINTER(i32)]
    lib.gdr_profile_end.restype = i32
    lib.gdr_gate_status.argtypes = [dp, ctypes.c_int64, p, sz, p, p]
    lib.gdr_gate_status.restype = i32
    lib.gdr_set_local_form.argtypes = [i32]
    lib.gdr_set_local_form.restype = i32
    lib.gdr_set_walk_levels.argtypes = [i32]
    lib.gdr_set_walk_levels.restype = i32
    lib.gdr_status_string.argtypes = [i32]
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_last_error.argtypes = []
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_version.argtypes = []
    lib.gdr_version.restype = i32
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise GdrError(rc, load().gdr_last_error().decode())


def _policy(policy) -> int:
    if policy in (RECOMPUTE, "recompute", "R"):
        return RECOMPUTE
    if policy in (FULL_SAVE, "full_save", "A"):
        return FULL_SAVE
    raise ValueError(f"unknown policy {policy!r}")


def make_desc(B, T, H, gate, dtype, DK=128, DV=128, C=64) -> Desc:
    return Desc(B, T, H, DK, DV, C, gate, dtype)


def workspace_size(B, T, H, gate="scalar", dtype="bf16", policy="recompute", n_seq=None,
                   DK=128, DV=128):
    """(saved_bytes, scratch_bytes) for a problem; gate "scalar", "vector",
    "none" (DeltaNet) or "gdn2"; n_seq: sequences of a packed variable-length
    batch (B = 1), None for a regular batch."""
    kind = {"scalar": GATE_SCALAR, "vector": GATE_VECTOR, "none": GATE_NONE, "gdn2": GATE_GDN2}[gate]
    d = make_desc(B, T, H, kind, DT_F32 if dtype == "fp32" else DT_BF16, DK=DK, DV=DV)
    return _sizes(d, _policy(policy), n_seq)


def _sizes(d, pol, n_seq):
    sv, sc = ctypes.c_size_t(), ctypes.c_size_t()
    lib = load()
    if n_seq is None:
        _check(lib.gdr_workspace_size(ctypes.byref(d), pol, ctypes.byref(sv), ctypes.byref(sc)))
    else:
        _check(lib.gdr_workspace_size_varlen(ctypes.byref(d), n_seq, pol, ctypes.byref(sv),
                                             ctypes.byref(sc)))
    return sv.value, sc.value


def profile_begin(max_launches: int = 4096):
    """Start per-stage event timing of every launch the library makes."""
    _check(load().gdr_profile_begin(max_launches))


def profile_end() -> dict:
    """Stop timing; returns {stage: (launches, total_ms)} (waits for the GPU)."""
    arr = (StageTime * 16)()
    n = ctypes.c_int()
    _check(load().gdr_profile_end(arr, 16, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


GATE_POSITIVE, GATE_RANGE, GATE_NONFINITE = 1, 2, 4


def gate_status(q, g, v, scratch, n_seq=None, status=None):
    """Gate-check bits of the last call that ran with this problem and this
    scratch (GATE_POSITIVE | GATE_RANGE | GATE_NONFINITE; 0 = in contract),
    as a device int32 tensor written on the current stream (no sync here)."""
    torch = _torch()
    d = _desc_from(q, g, v)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=q.device)
    _check(load().gdr_gate_status(ctypes.byref(d), -1 if n_seq is None else n_seq, _ptr(scratch),
                                  scratch.numel(), _ptr(status), _stream()))
    return status


def set_local_form(form: str) -> str:
    """Launch form of the scalar-gate three-product local backward:
    "persistent" (default) or "per_chunk" (one workgroup per chunk and head,
    the form of the seven-product kernel). Returns the previous form."""
    forms = {"persistent": 0, "per_chunk": 1}
    if form not in forms:
        raise ValueError(f"unknown form {form!r}")
    rc = load().gdr_set_local_form(forms[form])
    if rc < 0:
        _check(rc)
    return {v: k for k, v in forms.items()}[rc]


def set_walk_levels(form: str) -> str:
    """Form of the state walks: "auto" (default: segmented, two-level walks
    where a one-level launch would leave most compute units idle) or "one"
    (every walk start to end). Returns the previous form."""
    forms = {"auto": 0, "one": 1}
    if form not in forms:
        raise ValueError(f"unknown form {form!r}")
    rc = load().gdr_set_walk_levels(forms[form])
    if rc < 0:
        _check(rc)
    return {v: k for k, v in forms.items()}[rc]


# ---------------------------------------------------------------- torch side

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _desc_from(q, g, v):
    torch = _torch()
    B, T, H, DK = q.shape
    DV = v.shape[-1]
    gate = GATE_NONE if g is None else GATE_VECTOR if g.dim() == 4 else GATE_SCALAR
    if q.dtype == torch.bfloat16:
        dt = DT_BF16
    elif q.dtype == torch.float32:
        dt = DT_F32
    else:
        raise TypeError(f"q dtype {q.dtype}: expected bfloat16 or float32")
    return make_desc(B, T, H, gate, dt, DK=DK, DV=DV)


def _validate(q, k, v, g, beta, n_seq=None, *, h0=None, dO=None, dht=None, out=None,
              saved=None, saved_bytes=0, scratch=None, erase=None, write=None, o=None):
    """Checks every tensor against the problem q and v define before any
    pointer reaches the library: device (one device, all of them), layout
    (contiguous), exact shape against (B, T, H, DK, DV) and the state count
    (B, or n_seq for a packed batch), and dtype (q's for the token tensors,
    float32 for g and the states, uint8 for the workspaces)."""
    torch = _torch()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError(f"q and v must be [B,T,H,D], got {tuple(q.shape)} and {tuple(v.shape)}")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q dtype {q.dtype}: expected bfloat16 or float32")
    B, T, H, DK = q.shape
    DV = v.shape[3]
    ns = B if n_seq is None else n_seq
    tok_k, tok_v, row = (B, T, H, DK), (B, T, H, DV), (B, T, H)
    state = (ns, H, DK, DV)
    f32 = torch.float32
    spec = [("q", q, tok_k, q.dtype), ("k", k, tok_k, q.dtype), ("v", v, tok_v, q.dtype),
            ("beta", beta, row, q.dtype), ("h0", h0, state, f32), ("dO", dO, tok_v, q.dtype),
            ("dht", dht, state, f32), ("o", o, tok_v, q.dtype)]
    if g is not None:
        if g.dim() == 3:
            spec.append(("g", g, row, f32))
        else:
            spec.append(("g", g, tok_k, f32))
    gdn2 = erase is not None or write is not None
    if gdn2:
        spec = [x for x in spec if x[0] != "beta"]
        spec += [("erase", erase, tok_k, q.dtype), ("write", write, tok_v, q.dtype)]
    if out is not None:
        spec += [("dq", out.get("dq"), tok_k, q.dtype), ("dk", out.get("dk"), tok_k, q.dtype),
                 ("dv", out.get("dv"), tok_v, q.dtype), ("dh0", out.get("dh0"), state, f32)]
        gate_grads = (("derase", tok_k), ("dwrite", tok_v)) if gdn2 else (("dbeta", row),)
        spec += [(n, out.get(n), shp, q.dtype) for n, shp in gate_grads]
        for name in ("dq", "dk", "dv") + tuple(n for n, _ in gate_grads):
            if out.get(name) is None:
                raise ValueError(f"out['{name}'] is required")
        if g is not None:
            if out.get("dg") is None:
                raise ValueError("out['dg'] is required when g is given")
            spec.append(("dg", out["dg"], tuple(g.shape), f32))
    if saved is not None:
        spec.append(("saved", saved, None, torch.uint8))
    if scratch is not None:
        spec.append(("scratch", scratch, None, torch.uint8))
    for name, t, shape, dtype in spec:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != dtype:
            raise TypeError(f"{name} dtype {t.dtype}: expected {dtype}")
        if shape is not None and tuple(t.shape) != shape:
            raise ValueError(f"{name} shape {tuple(t.shape)}: expected {shape}")
    if saved is not None and saved.numel() < saved_bytes:
        raise ValueError(f"saved holds {saved.numel()} bytes, {saved_bytes} needed")


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _scratch(nbytes, device):
    torch = _torch()
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _seqs(cu_seqlens, q):
    """Sequence count of a packed batch (None for a regular batch)."""
    torch = _torch()
    if cu_seqlens is None:
        return None
    if not cu_seqlens.is_cuda or cu_seqlens.dtype != torch.int64 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int64 device tensor")
    if not cu_seqlens.is_contiguous() or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be contiguous with n_seq + 1 >= 1 entries")
    if q.shape[0] != 1:
        raise ValueError(f"a packed batch has batch size 1, got {q.shape[0]}")
    return cu_seqlens.numel() - 1


def gdr_fwd(q, k, v, g, beta, h0=None, policy="recompute", want_ht=True, scratch=None,
            cu_seqlens=None, o=None):
    """Forward. Returns (o, ht or None, saved or None).

    cu_seqlens (int64 device tensor of n_seq + 1 token offsets) makes the
    single row of q (batch size 1) a packed batch of n_seq sequences, each
    with its own state: h0 and ht are then [n_seq, H, DK, DV]. o: an output
    tensor shaped like v to write into (a new one by default); the rows of
    tokens outside every sequence keep their contents."""
    torch = _torch()
    n_seq = _seqs(cu_seqlens, q)
    _validate(q, k, v, g, beta, n_seq, h0=h0, scratch=scratch, o=o)
    d = _desc_from(q, g, v)
    pol = _policy(policy)
    lib = load()
    saved_b, scratch_b = _sizes(d, pol, n_seq)
    B, T, H, _ = q.shape
    ns = B if n_seq is None else n_seq
    if o is None:
        o = torch.empty_like(v)
    ht = torch.empty((ns, H, q.shape[-1], v.shape[-1]), dtype=torch.float32,
                     device=q.device) if want_ht else None
    saved = torch.empty(saved_b, dtype=torch.uint8, device=q.device) if saved_b else None
    if scratch is None:
        scratch = _scratch(scratch_b, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht),
            _ptr(saved), _ptr(scratch), scratch.numel(), _stream())
    if n_seq is None:
        _check(lib.gdr_fwd(ctypes.byref(d), pol, *args))
    else:
        _check(lib.gdr_fwd_varlen(ctypes.byref(d), pol, _ptr(cu_seqlens), n_seq, *args))
    return o, ht, saved


def _bwd(name, q, k, v, g, beta, h0, dO, dht, saved, policy, want_dh0, scratch, out,
         cu_seqlens=None):
    torch = _torch()
    n_seq = _seqs(cu_seqlens, q)
    if dO is None:
        raise ValueError("dO is required")
    d = _desc_from(q, g, v)
    pol = _policy(policy)
    lib = load()
    saved_b, scratch_b = _sizes(d, pol, n_seq)
    if pol == FULL_SAVE and saved is None:
        raise ValueError("the full-save backward needs the forward's saved area")
    _validate(q, k, v, g, beta, n_seq, h0=h0, dO=dO, dht=dht, out=out, saved=saved,
              saved_bytes=saved_b, scratch=scratch)
    B, T, H, _ = q.shape
    ns = B if n_seq is None else n_seq
    if out is None:
        out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                   dg=None if g is None else torch.empty_like(g), dbeta=torch.empty_like(beta),
                   dh0=torch.empty((ns, H, q.shape[-1], v.shape[-1]), dtype=torch.float32,
                                   device=q.device)
                   if want_dh0 else None)
    if scratch is None:
        scratch = _scratch(scratch_b, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(dO), _ptr(dht),
            _ptr(saved), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out.get("dg")),
            _ptr(out["dbeta"]), _ptr(out.get("dh0")), _ptr(scratch), scratch.numel(), _stream())
    if n_seq is None:
        _check(getattr(lib, name)(ctypes.byref(d), pol, *args))
    elif name == "gdr_bwd":
        _check(lib.gdr_bwd_varlen(ctypes.byref(d), pol, _ptr(cu_seqlens), n_seq, *args))
    else:
        raise ValueError(f"{name} has no packed-batch form")
    return out


def gdr_bwd(q, k, v, g, beta, h0, dO, dht=None, saved=None, policy="recompute",
            want_dh0=True, scratch=None, out=None, cu_seqlens=None):
    """Backward (ReWY producer). Returns dict dq, dk, dv, dg, dbeta, dh0.
    cu_seqlens as for gdr_fwd (the same offsets the forward ran with)."""
    return _bwd("gdr_bwd", q, k, v, g, beta, h0, dO, dht, saved, policy, want_dh0, scratch,
                out, cu_seqlens)


def gdr_fwd_gdn2(q, k, v, g, erase, write, h0=None, policy="recompute", want_ht=True,
                 scratch=None, cu_seqlens=None, o=None):
    """GDN2 forward (per-key-channel gate g [B,T,H,DK] fp32, erase gate
    [B,T,H,DK] per key and write gate [B,T,H,DV] per value, bf16). Returns
    (o, ht, saved). cu_seqlens and o: as for gdr_fwd."""
    torch = _torch()
    if erase is None or write is None or g is None or g.dim() != 4:
        raise ValueError("GDN2 needs a per-channel g and both erase and write gates")
    n_seq = _seqs(cu_seqlens, q)
    _validate(q, k, v, g, None, n_seq, h0=h0, scratch=scratch, erase=erase, write=write, o=o)
    d = _desc_from(q, g, v)
    d.gate = GATE_GDN2
    pol = _policy(policy)
    lib = load()
    saved_b, scratch_b = _sizes(d, pol, n_seq)
    B, T, H, _ = q.shape
    ns = B if n_seq is None else n_seq
    if o is None:
        o = torch.empty_like(v)
    ht = torch.empty((ns, H, q.shape[-1], v.shape[-1]), dtype=torch.float32,
                     device=q.device) if want_ht else None
    saved = torch.empty(saved_b, dtype=torch.uint8, device=q.device) if saved_b else None
    if scratch is None:
        scratch = _scratch(scratch_b, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(erase), _ptr(write), _ptr(h0), _ptr(o), _ptr(ht),
            _ptr(saved), _ptr(scratch), scratch.numel(), _stream())
    if n_seq is None:
        _check(lib.gdr_fwd_gdn2(ctypes.byref(d), pol, *args))
    else:
        _check(lib.gdr_fwd_gdn2_varlen(ctypes.byref(d), pol, _ptr(cu_seqlens), n_seq, *args))
    return o, ht, saved


def gdr_bwd_gdn2(q, k, v, g, erase, write, h0, dO, dht=None, saved=None, policy="recompute",
                 want_dh0=True, scratch=None, out=None, cu_seqlens=None):
    """GDN2 backward. Returns dict dq, dk, dv, dg, derase, dwrite, dh0.
    cu_seqlens: the offsets the forward ran with (packed batch)."""
    torch = _torch()
    if erase is None or write is None or g is None or g.dim() != 4:
        raise ValueError("GDN2 needs a per-channel g and both erase and write gates")
    if dO is None:
        raise ValueError("dO is required")
    n_seq = _seqs(cu_seqlens, q)
    d = _desc_from(q, g, v)
    d.gate = GATE_GDN2
    pol = _policy(policy)
    lib = load()
    saved_b, scratch_b = _sizes(d, pol, n_seq)
    if pol == FULL_SAVE and saved is None:
        raise ValueError("the full-save backward needs the forward's saved area")
    _validate(q, k, v, g, None, n_seq, h0=h0, dO=dO, dht=dht, out=out, saved=saved,
              saved_bytes=saved_b, scratch=scratch, erase=erase, write=write)
    B, T, H, _ = q.shape
    ns = B if n_seq is None else n_seq
    if out is None:
        out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                   dg=torch.empty_like(g), derase=torch.empty_like(erase),
                   dwrite=torch.empty_like(write),
                   dh0=torch.empty((ns, H, q.shape[-1], v.shape[-1]), dtype=torch.float32,
                                   device=q.device) if want_dh0 else None)
    if scratch is None:
        scratch = _scratch(scratch_b, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(erase), _ptr(write), _ptr(h0), _ptr(dO), _ptr(dht),
            _ptr(saved), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
            _ptr(out["derase"]), _ptr(out["dwrite"]), _ptr(out.get("dh0")), _ptr(scratch),
            scratch.numel(), _stream())
    if n_seq is None:
        _check(lib.gdr_bwd_gdn2(ctypes.byref(d), pol, *args))
    else:
        _check(lib.gdr_bwd_gdn2_varlen(ctypes.byref(d), pol, _ptr(cu_seqlens), n_seq, *args))
    return out


def gdr_bwd_wy7(q, k, v, g, beta, h0, dO, dht=None, saved=None, policy="recompute",
                want_dh0=True, scratch=None, out=None):
    """Backward with the expanded seven-product WY producer (ablation)."""
    return _bwd("gdr_bwd_wy7", q, k, v, g, beta, h0, dO, dht, saved, policy, want_dh0,
                scratch, out)


# ------------------------------------------------------------- autograd

def _autograd_function():
    torch = _torch()

    class _ChunkGatedDeltaRule(torch.autograd.Function):
        """Forward by gdr_fwd, backward by gdr_bwd; no arithmetic here (the
        only torch work is making the incoming output adjoint contiguous)."""

        @staticmethod
        def forward(ctx, q, k, v, g, beta, h0, policy, cu_seqlens):
            ctx.set_materialize_grads(False)
            o, ht, saved = gdr_fwd(q, k, v, g, beta, h0, policy=policy, cu_seqlens=cu_seqlens)
            ctx.policy = policy
            ctx.has_g, ctx.has_h0 = g is not None, h0 is not None
            ctx.save_for_backward(q, k, v, g if g is not None else q.new_empty(0), beta,
                                  h0 if h0 is not None else q.new_empty(0),
                                  saved if saved is not None else q.new_empty(0, dtype=torch.uint8),
                                  cu_seqlens if cu_seqlens is not None else q.new_empty(0, dtype=torch.int64))
            ctx.has_saved, ctx.packed = saved is not None, cu_seqlens is not None
            return o, ht

        @staticmethod
        def backward(ctx, dO, dht):
            q, k, v, g, beta, h0, saved, cu = ctx.saved_tensors
            g = g if ctx.has_g else None
            h0 = h0 if ctx.has_h0 else None
            saved = saved if ctx.has_saved else None
            cu = cu if ctx.packed else None
            if dO is None and dht is None:
                return (None,) * 8
            if dO is None:
                dO = torch.zeros_like(v)
            gr = gdr_bwd(q, k, v, g, beta, h0, dO.contiguous(),
                         None if dht is None else dht.contiguous(), saved=saved,
                         policy=ctx.policy, want_dh0=h0 is not None, cu_seqlens=cu)
            return (gr["dq"], gr["dk"], gr["dv"], gr["dg"], gr["dbeta"], gr["dh0"], None, None)

    return _ChunkGatedDeltaRule


def _autograd_gdn2():
    torch = _torch()

    class _ChunkGDN2(torch.autograd.Function):
        """GDN2 forward by gdr_fwd_gdn2, backward by gdr_bwd_gdn2; no arithmetic
        here (an absent output adjoint is passed as zeros)."""

        @staticmethod
        def forward(ctx, q, k, v, g, erase, write, h0, policy, cu_seqlens):
            ctx.set_materialize_grads(False)
            o, ht, saved = gdr_fwd_gdn2(q, k, v, g, erase, write, h0, policy=policy,
                                        cu_seqlens=cu_seqlens)
            ctx.policy = policy
            ctx.has_h0 = h0 is not None
            ctx.has_saved, ctx.packed = saved is not None, cu_seqlens is not None
            ctx.save_for_backward(q, k, v, g, erase, write,
                                  h0 if h0 is not None else q.new_empty(0),
                                  saved if saved is not None else q.new_empty(0, dtype=torch.uint8),
                                  cu_seqlens if cu_seqlens is not None else q.new_empty(0, dtype=torch.int64))
            return o, ht

        @staticmethod
        def backward(ctx, dO, dht):
            q, k, v, g, erase, write, h0, saved, cu = ctx.saved_tensors
            h0 = h0 if ctx.has_h0 else None
            saved = saved if ctx.has_saved else None
            cu = cu if ctx.packed else None
            if dO is None and dht is None:
                return (None,) * 9
            if dO is None:
                dO = torch.zeros_like(v)
            gr = gdr_bwd_gdn2(q, k, v, g, erase, write, h0, dO.contiguous(),
                              None if dht is None else dht.contiguous(), saved=saved,
                              policy=ctx.policy, want_dh0=h0 is not None, cu_seqlens=cu)
            return (gr["dq"], gr["dk"], gr["dv"], gr["dg"], gr["derase"], gr["dwrite"], gr["dh0"],
                    None, None)

    return _ChunkGDN2


_AUTOGRAD = None
_AUTOGRAD_GDN2 = None


def chunk_gdn2(q, k, v, g, erase, write, h0=None, policy="recompute", cu_seqlens=None):
    """Differentiable GDN2 operator (per-key-channel decay g, erase gate per
    key channel, write gate per value channel; bf16 q, k, v, erase, write):
    returns (o, ht) and back-propagates through gdr_bwd_gdn2 into q, k, v,
    g, erase, write and h0. cu_seqlens makes a packed batch."""
    global _AUTOGRAD_GDN2
    if _AUTOGRAD_GDN2 is None:
        _AUTOGRAD_GDN2 = _autograd_gdn2()
    return _AUTOGRAD_GDN2.apply(q, k, v, g, erase, write, h0, policy, cu_seqlens)


def chunk_gated_delta_rule(q, k, v, g, beta, h0=None, policy="recompute", cu_seqlens=None):
    """Differentiable operator: returns (o, ht) and back-propagates through
    the library's backward into q, k, v, g, beta and h0. g None is DeltaNet
    (no decay); cu_seqlens makes a packed batch. policy "full_save" keeps the
    forward's chunk quantities for the backward instead of recomputing them."""
    global _AUTOGRAD
    if _AUTOGRAD is None:
        _AUTOGRAD = _autograd_function()
    return _AUTOGRAD.apply(q, k, v, g, beta, h0, policy, cu_seqlens)
