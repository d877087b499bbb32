"""The C-ABI library loads, exports every function include/gdr.h declares, and
rejects invalid or unsupported calls before touching the device. No compute
calls are made here (no GPU needed)."""
import ctypes
import os
import re

import pytest

import delta_rule_linear_gdr_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gdr.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function():
    lib = gdr.load()
    names = _declared()
    assert set(names) == set(gdr.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def _desc(**kw):
    base = dict(B=1, T=128, H=2, gate=0, dtype=0)
    base.update(kw)
    return gdr.make_desc(base["B"], base["T"], base["H"], base["gate"], base["dtype"],
                         DK=base.get("DK", 128), DV=base.get("DV", 128), C=base.get("C", 64))


def _ws(d, policy=0):
    sv, sc = ctypes.c_size_t(), ctypes.c_size_t()
    rc = gdr.load().gdr_workspace_size(ctypes.byref(d) if d is not None else None, policy,
                                       ctypes.byref(sv), ctypes.byref(sc))
    return rc, sv.value, sc.value


def test_workspace_sizes():
    T64x128, T128x128, T64x64, GN = 16384, 32768, 8192, 512
    rc, sv, sc = _ws(_desc(T=8192, H=16), 0)
    assert rc == 0 and sv == 0
    # recompute: the backward holds the scan operands both directions read
    # (-W, Kt, gn: one orientation each), U for the forward scan, X and Y for
    # the reverse one, A^T and A, and the per-chunk h, R, dh, Rb of every
    # (chunk, head) (plus the 16 bytes of gate-check words of every (chunk, head))
    per = 2 * T64x128 + GN + T64x128 + 2 * T64x64 + T128x128 + T64x128 \
        + T64x128 + T128x128 + T128x128 + T64x128 + 16
    assert per == 213520
    assert sc == 2048 * per
    rc, sv, sc = _ws(_desc(T=8192, H=16), 1)
    assert rc == 0
    # full save keeps A^T, Kt, -W, gn, Hm^T, Qg^T, h, R (115,200 B per chunk-head),
    # which the forward's own scan reads too; the forward's scratch holds U,
    # Qg, Hm, the backward's X, Y, dh, Rb and A for the seven-product producer
    assert sv == 2048 * (T64x64 + 2 * T64x128 + GN + T64x64 + T64x128 + T128x128 + T64x128)
    assert sv == 2048 * 115200
    assert sc == 2048 * (16 + max(2 * T64x128 + T64x64, 2 * T64x128 + 2 * T128x128 + T64x64))


def test_workspace_two_level_walk_buffers():
    """A regular batch whose one-level walk launch would fill at most a
    quarter of 256 CUs, with walks long enough for 4 or more segments of at
    least 20 chunks, walks in segments. Its workspace adds, for both
    directions, each summarized segment's transfer map and zero-entry exit
    state (2 x 64 KiB per state entry) and each segment's entry state (64 KiB
    per state entry). At (1, 8192, 2) the recompute backward walks both
    directions in 5 segments; at (1, 8192, 4) the full-save backward's reverse
    walk takes 5, while the recompute pair would get only 3 and stays one-level
    (the forward's 5-segment buffers fit in the backward's larger scratch)."""
    T64x128, T128x128, T64x64, GN = 16384, 32768, 8192, 512
    state = 128 * 128 * 4

    def seg_bytes(nseg, nsh):
        return 2 * (nseg - 1) * nsh * 2 * state + 2 * nseg * nsh * state

    per = 2 * T64x128 + GN + T64x128 + 2 * T64x64 + T128x128 + T64x128 \
        + T64x128 + T128x128 + T128x128 + T64x128 + 16
    rc, sv, sc = _ws(_desc(T=8192, H=2), 0)
    assert rc == 0 and sv == 0
    assert sc == 256 * per + seg_bytes(5, 2)
    rc, sv, sc = _ws(_desc(T=8192, H=4), 1)
    assert rc == 0 and sv == 512 * 115200
    assert sc == 512 * (16 + 2 * T64x128 + 2 * T128x128 + T64x64) + seg_bytes(5, 4)
    rc, sv, sc = _ws(_desc(T=8192, H=4), 0)
    assert rc == 0 and sc == 512 * per
    # too short for four segments of twenty chunks: one level
    rc, sv, sc = _ws(_desc(T=4096, H=4), 1)
    assert rc == 0 and sc == 256 * (16 + 2 * T64x128 + 2 * T128x128 + T64x64)
    # sixteen heads fill the chip with one-level walks
    rc, sv, sc = _ws(_desc(T=8192, H=16), 0)
    assert rc == 0 and sc == 2048 * per


@pytest.mark.parametrize("kw,status", [
    (dict(DK=192), -2), (dict(DV=1025), -2), (dict(DK=192, DV=160), -2), (dict(DK=0), -1), (dict(DV=-3), -1), (dict(C=32), -2),
    (dict(gate=5), -1), (dict(gate=4), -1), (dict(dtype=7), -1), (dict(B=-1), -1),
])
def test_descriptor_validation(kw, status):
    rc, _, _ = _ws(_desc(**kw))
    assert rc == status
    assert gdr.load().gdr_last_error()


def test_ragged_length_sizes_whole_chunks():
    # T = 100: two chunks, the second holding 36 tokens; workspaces count tiles
    rc, sv100, sc100 = _ws(_desc(T=100), 1)
    assert rc == 0
    rc, sv128, sc128 = _ws(_desc(T=128), 1)
    assert rc == 0 and (sv100, sc100) == (sv128, sc128)
    rc, sv1, sc1 = _ws(_desc(T=1), 0)
    rc64, sv64, sc64 = _ws(_desc(T=64), 0)
    assert rc == 0 and rc64 == 0 and (sv1, sc1) == (sv64, sc64)


def test_null_descriptor_and_bad_policy():
    assert _ws(None)[0] == -1
    assert _ws(_desc(), policy=3)[0] == -1


def _fwd(d, **ptrs):
    lib = gdr.load()
    P = {n: ptrs.get(n) for n in ("q", "k", "v", "g", "beta", "h0", "o", "ht", "saved", "scratch")}
    return lib.gdr_fwd(ctypes.byref(d), ptrs.get("policy", 0), P["q"], P["k"], P["v"], P["g"],
                       P["beta"], P["h0"], P["o"], P["ht"], P["saved"], P["scratch"],
                       ptrs.get("scratch_bytes", 0), None)


def test_forward_rejects_null_and_small_workspace_without_launching():
    d = _desc()
    assert _fwd(d) == -1
    assert b"NULL" in gdr.load().gdr_last_error()
    fake = 1 << 20  # never dereferenced: validation fails first
    assert _fwd(d, q=fake, k=fake, v=fake, g=fake, beta=fake, o=fake, scratch=fake,
                scratch_bytes=16) == -3
    assert _fwd(d, q=fake + 8, k=fake, v=fake, g=fake, beta=fake, o=fake, scratch=fake,
                scratch_bytes=1 << 40) == -1
    assert _fwd(d, policy=1, q=fake, k=fake, v=fake, g=fake, beta=fake, o=fake, scratch=fake,
                scratch_bytes=1 << 40) == -1  # full save needs `saved`


def test_empty_problems_are_no_ops():
    assert _fwd(_desc(B=0)) == 0
    assert _fwd(_desc(H=0)) == 0
    assert _fwd(_desc(T=0)) == 0  # ht NULL: nothing to write


def test_status_strings():
    lib = gdr.load()
    for st in (0, -1, -2, -3, -4, 99):
        assert lib.gdr_status_string(st)


def _ws_varlen(d, n_seq, policy=0):
    sv, sc = ctypes.c_size_t(), ctypes.c_size_t()
    rc = gdr.load().gdr_workspace_size_varlen(ctypes.byref(d), n_seq, policy, ctypes.byref(sv),
                                              ctypes.byref(sc))
    return rc, sv.value, sc.value


def test_packed_workspace_counts_slots_and_tables():
    """A packed batch of n sequences over T tokens has at most ceil(T/64) + n
    chunks per head; the workspace holds that many tiles (each tile kind in
    its own 256-byte-aligned block, as for a regular row of that many chunks)
    plus the offsets, the per-sequence table, the per-slot table and the
    longest-first sequence order. (Sixteen heads: the regular row's walks are
    then one-level, with no segment buffers; packed batches always walk in
    one level.)"""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for T, n in ((8192, 7), (100, 3), (64, 0), (1, 1)):
        for pol in (0, 1):
            nslot = (T + 63) // 64 + n
            rc, sv, sc = _ws_varlen(_desc(T=T, H=16), n, pol)
            assert rc == 0
            # a regular row with nslot chunks has exactly the tile part
            rc, sv_r, sc_r = _ws(_desc(T=64 * nslot, H=16), pol)
            assert rc == 0
            assert sv == sv_r
            assert sc == sc_r + al(8 * (n + 1)) + al(8 * n) + al(8 * nslot) + al(4 * n)


def test_packed_validation_without_launching():
    lib = gdr.load()
    assert _ws_varlen(_desc(B=2), 3)[0] == -1            # sequences live along T
    assert _ws_varlen(_desc(), -1)[0] == -1
    assert _ws_varlen(_desc(DK=192), 2)[0] == -2
    assert _ws_varlen(_desc(T=1 << 31), 2)[0] == -2       # the slot table holds 32-bit token indices
    assert _ws_varlen(_desc(T=(1 << 31) - 64), 2)[0] == 0
    fake = 1 << 20  # never dereferenced: validation fails first
    d = _desc(T=256)
    sc = _ws_varlen(d, 2)[2]

    def fwd(cu, n=2, nbytes=sc, **p):
        P = {x: p.get(x, fake) for x in ("q", "k", "v", "g", "beta", "o", "scratch")}
        return lib.gdr_fwd_varlen(ctypes.byref(d), 0, cu, n, P["q"], P["k"], P["v"], P["g"],
                                  P["beta"], None, P["o"], None, None, P["scratch"], nbytes,
                                  None)

    assert fwd(None) == -1
    assert b"cu_seqlens" in lib.gdr_last_error()
    assert fwd(fake + 4) == -1                            # not 8-byte aligned
    assert fwd(fake, nbytes=sc // 4) == -3                # tables + tiles do not fit
    assert fwd(fake, q=None) == -1
    assert fwd(fake, n=-2) == -1
    # no sequences, or no tokens with no state to pass through: nothing to do
    assert fwd(fake, n=0) == 0
    d0 = _desc(T=0)
    assert lib.gdr_fwd_varlen(ctypes.byref(d0), 0, fake, 3, None, None, None, None, None, None,
                              None, None, None, None, 0, None) == 0
    P = [None] * 16
    assert lib.gdr_bwd_varlen(ctypes.byref(_desc(B=2)), 0, fake, 1, *P, 0, None) == -1
    assert lib.gdr_bwd_varlen(ctypes.byref(d), 0, None, 1, *P, 0, None) == -1


def test_no_gate_workspace_and_null_gate():
    """DeltaNet (gate kind 2): the scalar-gate workspace plus a zero log-decay
    array and a sink for its gradient; g may be NULL."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for T, H in ((8192, 16), (100, 3)):
        for pol in (0, 1):
            rc, sv, sc = _ws(_desc(T=T, H=H, gate=2), pol)
            rc2, sv2, sc2 = _ws(_desc(T=T, H=H, gate=0), pol)
            assert rc == 0 and rc2 == 0
            assert sv == sv2 and sc == sc2 + 2 * al(4 * T * H)
    fake = 1 << 20  # never dereferenced: validation fails first
    d = _desc(gate=2)
    # g NULL passes validation; the too-small workspace is what fails
    assert _fwd(d, q=fake, k=fake, v=fake, beta=fake, o=fake, scratch=fake, scratch_bytes=16) == -3
    assert _fwd(_desc(gate=0), q=fake, k=fake, v=fake, beta=fake, o=fake, scratch=fake,
                scratch_bytes=16) == -1


@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("dk,dv", [(80, 112), (96, 80), (128, 64)])
def test_narrow_widths_workspace(gate, dk, dv):
    """Widths below 128: the 128-wide workspace plus zero-padded copies of the
    token tensors (q, k, v, o or dO, dq, dk, dv at 128 wide), of a vector gate
    and its gradient, and of three states."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    B, T, H = 2, 100, 3
    for pol in (0, 1):
        for dtype, esz in ((0, 2), (1, 4)):
            rc, sv, sc = _ws(_desc(B=B, T=T, H=H, gate=gate, dtype=dtype, DK=dk, DV=dv), pol)
            rc2, sv2, sc2 = _ws(_desc(B=B, T=T, H=H, gate=gate, dtype=dtype), pol)
            assert rc == 0 and rc2 == 0 and sv == sv2
            rows = B * T * H
            pad = 7 * al(rows * 128 * esz) + 3 * al(B * H * 128 * 128 * 4)
            if gate == 1:
                pad += 2 * al(rows * 128 * 4)
            assert sc == sc2 + pad


def test_noalloc_rejects_problems_past_its_array():
    """gdr_bwd_noalloc refuses, before any device call, a problem whose
    scratch exceeds the library's fixed array (GDR_NOALLOC_SCRATCH_MAX)."""
    src = open(os.path.join(ROOT, "include", "gdr.h")).read()
    m = re.search(r"#define GDR_NOALLOC_SCRATCH_MAX \(\(size_t\)(\d+) << (\d+)\)", src)
    cap = int(m.group(1)) << int(m.group(2))
    lib = gdr.load()
    fits = _desc(T=2048, H=9)
    too_big = _desc(T=2048, H=10)
    assert _ws(fits)[2] <= cap < _ws(too_big)[2]
    rc = lib.gdr_bwd_noalloc(ctypes.byref(too_big), 0, *([None] * 15), None)
    assert rc == -2 and b"fixed" in lib.gdr_last_error()
    rc = lib.gdr_bwd_noalloc(ctypes.byref(_desc(DK=200)), 0, *([None] * 15), None)
    assert rc == -2


def test_gdn2_entry_points_take_only_gdn2():
    """GDN2 goes through gdr_fwd_gdn2 / gdr_bwd_gdn2 alone; they take bf16
    inputs and refuse other gate kinds, all before any launch."""
    lib = gdr.load()
    nul = [None] * 20
    gd2 = _desc(gate=3)
    # the beta entry points refuse the GDN2 gate kind
    assert lib.gdr_fwd(ctypes.byref(gd2), 0, *nul[:10], 0, None) == -1
    assert lib.gdr_bwd(ctypes.byref(gd2), 0, *nul[:16], 0, None) == -1
    assert b"gdr_fwd_gdn2" in lib.gdr_last_error()
    # the GDN2 entry points refuse other gate kinds, fp32 and narrow widths
    for kw, status in ((dict(gate=1), -1), (dict(gate=3, dtype=1), -2), (dict(gate=3, DK=192), -2)):
        d = _desc(**kw)
        assert lib.gdr_fwd_gdn2(ctypes.byref(d), 0, *nul[:11], 0, None) == status, kw
        assert lib.gdr_bwd_gdn2(ctypes.byref(d), 0, *nul[:18], 0, None) == status, kw
    # a GDN2 descriptor without its gate tensors is refused
    assert lib.gdr_fwd_gdn2(ctypes.byref(gd2), 0, *nul[:11], 0, None) == -1
    # the workspace is the vector gate's
    assert _ws(gd2, 0) == _ws(_desc(gate=1), 0)
    assert _ws(gd2, 1) == _ws(_desc(gate=1), 1)


def test_gate_status_validates_before_any_launch():
    lib = gdr.load()
    d = _desc(T=256, gate=1)
    st = ctypes.c_void_p(64)  # never dereferenced: every case fails validation first
    assert lib.gdr_gate_status(ctypes.byref(d), -1, None, 0, st, None) == -1
    assert lib.gdr_gate_status(ctypes.byref(d), -1, ctypes.c_void_p(256), 1 << 30, None, None) == -1
    assert lib.gdr_gate_status(ctypes.byref(d), -1, ctypes.c_void_p(256), 64, st, None) == -3
    assert lib.gdr_gate_status(ctypes.byref(_desc(B=2)), 3, ctypes.c_void_p(256), 1 << 30, st,
                               None) == -1  # a packed batch has B = 1


def test_wide_values_run_as_value_blocks():
    """A value width above 128 runs as ceil(DV / 128) value blocks of the
    128-wide path: one saved area per block, scratch for the padded copies."""
    rc, sv128, sc128 = _ws(_desc(T=256, DV=128), 1)
    rc2, sv160, sc160 = _ws(_desc(T=256, DV=160), 1)
    rc3, sv300, _ = _ws(_desc(T=256, DV=300), 1)
    assert rc == rc2 == rc3 == 0
    assert sv160 == 2 * sv128 and sv300 == 3 * sv128
    assert sc160 > sc128
