"""Host-side checks of the tile layouts the kernels exchange (no GPU): the
scans' transposed fragment reads, the local backward's D / Hb tiles read
back transposed, and the transposed tiles (ttiles) the scans write for it.

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


# ---------------------------------------------------------------------------
# The local backward's D and Hb tiles: written with st_half_tr (lane l's half
# slot at position tr_slot(l)) and read back transposed by ld_frag_t64x64.

def ld_frag_t64x64(img, mt, ks):
    lo_addr, hi_addr = [], []
    for l in range(64):
        r, g = l & 15, l >> 4
        slot = tr_slot(4 * g + (r >> 2) + 16 * (r & 3))
        byte = (2 * ks * 2 + (mt >> 1)) * 1024 + slot * 16 + 8 * (mt & 1)
        lo_addr.append(byte // 2)
        hi_addr.append((byte + 2 * 1024) // 2)
    return np.concatenate([tr_read(img, lo_addr), tr_read(img, hi_addr)], axis=1)


def test_transposed_reads_of_64x64_tiles():
    X = np.arange(64 * 64, dtype=np.int32).reshape(64, 64) + 7
    img = lds_image(frag_tiles(X))  # 8 tiles, (m, k) at m * 2 + k
    want = frag_tiles(np.ascontiguousarray(X.T))
    for mt in range(4):
        for ks in range(2):
            assert np.array_equal(ld_frag_t64x64(img, mt, ks), want[mt * 2 + ks]), (mt, ks)


def test_half_slot_writes_place_whole_tiles():
    """st_half_tr: the epilogue of tile (ti, tj) writes, from lane (r, g), the
    four values X[16 tj + r][16 ti + 4 g + e] (row block tj, column block ti
    of the stored M = j, K = i matrix) into half ti & 1 of frag tile
    (tj, ti >> 1) at position tr_slot(lane); every such write together is
    the tr_slot image of the matrix's frag tiles."""
    X = np.arange(64 * 64, dtype=np.int32).reshape(64, 64) - 100
    img = np.zeros(8 * 512, np.int32)
    for ti in range(4):
        for tj in range(4):
            tile = tj * 2 + (ti >> 1)
            for lane in range(64):
                r, g = lane & 15, lane >> 4
                p = tile * 512 + tr_slot(lane) * 8 + 4 * (ti & 1)
                img[p:p + 4] = [X[16 * tj + r, 16 * ti + 4 * g + e] for e in range(4)]
    assert np.array_equal(img, lds_image(frag_tiles(X)))


# ---------------------------------------------------------------------------
# ttiles: the scans write h, dh and R transposed within each 16 x 16 tile by
# an MFMA with the identity; two of a lane's tile pieces side by side are a
# frag slab, which the local kernel takes as an operand as read.

def mfma_16x16x32(A_lanes, B_lanes):
    """v_mfma_f32_16x16x32_bf16 lane rule: lane (r, g) passes A[r][pik(g, j)]
    and B[pik(g, j)][r] in slot j; element i of lane (r, g) is C[4 g + i][r]."""
    A = np.zeros((16, 32)); B = np.zeros((32, 16))
    for lane in range(64):
        r, g = lane & 15, lane >> 4
        for j in range(8):
            A[r, pik(g, j)] = A_lanes[lane][j]
            B[pik(g, j), r] = B_lanes[lane][j]
    C = A @ B
    return [[C[4 * (lane >> 4) + i, lane & 15] for i in range(4)] for lane in range(64)]


def ident_pi(parity):
    return [[1.0 if pik(lane >> 4, j) == 16 * parity + (lane & 15) else 0.0 for j in range(8)]
            for lane in range(64)]


def ttile(X, mt, nt):
    return [[X[16 * mt + (lane & 15), 16 * nt + 4 * (lane >> 4) + i] for i in range(4)] for lane in range(64)]


def test_state_slab_times_identity_is_the_ttile():
    """The forward and reverse walks hold, per compute wave w and value tile u,
    the state's accumulator tiles S[key 32 w + 16 m + 4 g + i][value 16 u + r]
    (m = 0, 1); pack_pi of the two is a frag with M = values, K = keys, and
    its product with the identity of key half m is ttile (2 w + m, u)."""
    rng = np.random.default_rng(0)
    S = rng.standard_normal((128, 32))  # keys x (two value tiles)
    for w in range(4):
        for u in range(2):
            acc = [[[S[32 * w + 16 * m + 4 * (lane >> 4) + i, 16 * u + (lane & 15)] for i in range(4)]
                    for lane in range(64)] for m in range(2)]
            sfrag = [acc[0][lane] + acc[1][lane] for lane in range(64)]
            for m in range(2):
                got = mfma_16x16x32(sfrag, ident_pi(m))
                assert np.allclose(got, ttile(S, 2 * w + m, u)), (w, u, m)


def test_correction_tile_times_identity_is_the_ttile():
    """R: the walk's Z accumulator Z[row 16 w + 4 g + i][value 16 u + r], in
    the first half of an otherwise zero slab, times the identity of half 0."""
    rng = np.random.default_rng(1)
    Z = rng.standard_normal((64, 32))
    for w in range(4):
        for u in range(2):
            z4 = [[Z[16 * w + 4 * (lane >> 4) + i, 16 * u + (lane & 15)] for i in range(4)] for lane in range(64)]
            got = mfma_16x16x32([z + [0.0] * 4 for z in z4], ident_pi(0))
            assert np.allclose(got, ttile(Z, w, u)), (w, u)


def test_two_ttile_pieces_are_a_frag_slab():
    X = np.arange(48 * 64, dtype=np.int32).reshape(48, 64)
    frags = frag_tiles(X)  # tiles (mt, ks) at mt * 2 + ks
    for mt in range(3):
        for ks in range(2):
            lo, hi = ttile(X, mt, 2 * ks), ttile(X, mt, 2 * ks + 1)
            got = np.array([lo[lane] + hi[lane] for lane in range(64)])
            assert np.array_equal(got, frags[mt * 2 + ks]), (mt, ks)
