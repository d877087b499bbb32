"""Host-side check of the scans' transposed fragment reads (no GPU).

The reverse scan reads -W^T and the forward scan Kt^T as MFMA fragments
taken from the frag tiles of -W and Kt themselves, through gfx950's
transposing LDS read. This test emulates that read on the CPU -- the lane
rule of ds_read_b64_tr_b16 as measured on the device: within each group of
16 lanes, lane j receives as its element e the element j & 3 of the four
16-bit values lane 4 e + (j >> 2) loaded -- over the frag layout (kernels.h)
with the slot placement tr_slot, at the addresses ld_frag_t64x128 forms,
and checks every lane receives X^T's frag tile (mt, ks)."""
import numpy as np


def pik(g, j):
    return 4 * g + j if j < 4 else 12 + 4 * g + j


def tr_slot(s):
    return s ^ ((s >> 2) & 12)


def frag_tiles(X):
    """Frag layout of an M x K matrix: tile (mt, ks) at mt * (K / 32) + ks,
    lane (r, g) slot j = X[16 mt + r][32 ks + pik(g, j)]."""
    M, K = X.shape
    nk = K // 32
    out = np.zeros((M // 16 * nk, 64, 8), X.dtype)
    for mt in range(M // 16):
        for ks in range(nk):
            for lane in range(64):
                r, g = lane & 15, lane >> 4
                for j in range(8):
                    out[mt * nk + ks, lane, j] = X[16 * mt + r, 32 * ks + pik(g, j)]
    return out


def lds_image(tiles):
    """The scan ring's copy: 16-byte slot s of each tile at position tr_slot(s),
    as 16-bit words (8 per slot)."""
    img = np.zeros(tiles.shape[0] * 512, tiles.dtype)
    for t in range(tiles.shape[0]):
        for s in range(64):
            p = t * 512 + tr_slot(s) * 8
            img[p:p + 8] = tiles[t, s]
    return img


def tr_read(img, addr_words):
    """ds_read_b64_tr_b16 over 64 lanes; addr_words[l]: lane l's address in
    16-bit words."""
    loaded = np.stack([img[a:a + 4] for a in addr_words])  # [64][4]
    out = np.zeros_like(loaded)
    for l in range(64):
        grp, j = l >> 4, l & 15
        for e in range(4):
            out[l, e] = loaded[16 * grp + 4 * e + (j >> 2), j & 3]
    return out


def ld_frag_t(img, mt, ks):
    lo_addr, hi_addr = [], []
    for l in range(64):
        r, g = l & 15, l >> 4
        slot = tr_slot(4 * g + (r >> 2) + 16 * (r & 3))
        byte = (2 * ks * 4 + (mt >> 1)) * 1024 + slot * 16 + 8 * (mt & 1)
        lo_addr.append(byte // 2)
        hi_addr.append((byte + 4 * 1024) // 2)
    return np.concatenate([tr_read(img, lo_addr), tr_read(img, hi_addr)], axis=1)


def test_tr_slot_is_a_conflict_free_involution():
    perm = [tr_slot(s) for s in range(64)]
    assert sorted(perm) == list(range(64))
    assert all(tr_slot(tr_slot(s)) == s for s in range(64))
    for a in range(4):  # plain 16-byte reads: 16 lanes on 16 distinct slot positions mod 16
        assert len({tr_slot(16 * a + b) % 16 for b in range(16)}) == 16
    for g in range(4):  # transposed reads: the same per 16-lane group
        assert len({tr_slot(4 * g + (r >> 2) + 16 * (r & 3)) % 16 for r in range(16)}) == 16


def test_transposed_reads_give_the_transposes_frag_tiles():
    X = np.arange(64 * 128, dtype=np.int32).reshape(64, 128)  # distinct entries
    img = lds_image(frag_tiles(X))
    want = frag_tiles(np.ascontiguousarray(X.T))  # 128 x 64: tiles (mt, ks) at mt * 2 + ks
    for mt in range(8):
        for ks in range(2):
            got = ld_frag_t(img, mt, ks)
            assert np.array_equal(got, want[mt * 2 + ks]), (mt, ks)
