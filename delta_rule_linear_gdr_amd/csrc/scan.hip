// Inter-chunk state scans of the chunkwise gated delta rule.
//
// ReWY paper (paperpeel.com/paper/2611.01940), Sec. 2.1 and Sec. 3.5: the
// state scan is serial across chunks and parallel across value columns.
// One workgroup owns 16 (or 32) value columns of one head and walks the
// chunks; its four compute waves hold the 128 x 16 fp32 state per value
// tile, wave w owning key rows [32 w, 32 w + 32) as two accumulator tiles.
//
// Both directions run the same two-product step (the chunk system of Sec.
// 2.3, M R = Z - E S with W = A E and U = A Z, as the onedev.kr summary
// writes it in "How it works"):
//   forward, chunk c = 0 .. NT-1, state S = h_c:
//     Z = U - W S            (the correction R_c)
//     O = Qg S + Hm Z        (optional output)
//     S <- diag(gn) S + Kt^T Z
//   reverse, chunk c = NT-1 .. 0, state Sb = adjoint of the state at the end
//   of chunk c (output and next-state adjoints are summed before the local
//   pullback, paper Sec. 3.1 "State and gate composition"):
//     Z = Hm^T dO + Kt Sb    (the correction adjoint Rb_c)
//     Sb <- diag(gn) Sb + Qg^T dO - W^T Z
// Per step: A1 (16 x 128 per wave) times the state slabs, then A2 (32 x 64
// per wave) times the Z slabs. The chunk operands arrive pre-swizzled in
// frag/ctile order (kernels.h). -W and Kt are stored once each: A1 is one
// of them and A2 the transpose of the other, read from its frag tiles with
// LDS transpose reads (ld_frag_t64x128). The only on-chip exchange is the
// state and Z slabs through LDS (one 16-byte write and a few 16-byte reads
// per lane, two barriers). Every launch uses the loader-fed form below; in
// the forward launch the loader waves also form the output O.
// Parallelism is one serial walk ("chain") per (sequence, head, value
// slice, direction); see chain_of_block for how workgroups map onto chains.
// Every slice of a head reads the head's whole A1 and A2 (32 KiB per step),
// so the step time is set by each CU's L2-to-CU stream and by HBM rather
// than by the arithmetic.
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int NVS = DVD / 16;  // 16-column value tiles per head

// The chain a scan workgroup walks: sequence n (state entry), head hd, value
// slice vs (NV consecutive value tiles), direction, and the segment of the
// walk (two-level walks; 0 otherwise).
struct Chain {
    int64_t n, hd;
    int vs;
    bool bwd;
    int sg;
};

// Workgroups are dealt to the eight XCDs round-robin by index (block b runs
// on XCD b % 8). Chain groups -- the nvs slices of one (sequence, head,
// direction) -- are numbered J = 0, 1, ... and group J goes whole to XCD
// J % 8, so the slices of a group share their A1 / A2 tiles in that XCD's
// L2, and within an XCD the groups start in order of J. In a two-direction
// launch J alternates forward / reverse; the (sequence, head) pairs follow
// s.order (longest sequence first) in packed batches, so the longest walks
// start first. Workgroups past the last group (the grid is rounded up to
// whole rounds of eight groups) have no chain. With nseg segments per walk,
// a group is one segment of one walk, and consecutive groups are the
// segments of one walk.
__device__ __forceinline__ bool chain_of_block(const Shape& s, int nvs, int ndir, bool bwd1, int block,
                                               Chain& ch, int nseg = 1)
{
    const int x = block & 7, q = block >> 3;
    const int64_t J = (int64_t)(q / nvs) * 8 + x;
    if (J >= s.NS * s.H * ndir * nseg) return false;
    ch.vs = q % nvs;
    ch.sg = (int)(J % nseg);
    const int64_t J2 = J / nseg;
    ch.bwd = ndir == 2 ? (J2 & 1) != 0 : bwd1;
    const int64_t j = ndir == 2 ? J2 >> 1 : J2;
    const int64_t k = j / s.H;
    ch.hd = j % s.H;
    ch.n = s.order ? s.order[k] : k;
    return true;
}

unsigned scan_grid(const Shape& s, int nvs, int ndir, int nseg = 1)
{
    return (unsigned)((s.NS * s.H * ndir * nseg + 7) / 8 * 8 * nvs);
}

// ---------------------------------------------------------------------------
// Loader-fed form. Eight waves per workgroup: waves 0..3 run the step
// above; waves 4..7 move each step's operand tiles from global memory into
// a ring of three LDS slots,
// two steps ahead, with direct-to-LDS loads (global_load_lds_dwordx4: 64
// lanes x 16 B = one 1 KiB block per instruction, i.e. one frag tile or two
// ctiles, copied as is). The compute waves' instruction streams then carry
// no global loads, so a stall issuing loads behind the shared address unit
// no longer adds to the step's dependent chain (LDS exchange, MFMA,
// barrier).
//
// A workgroup owns NV consecutive 16-column value tiles. NV = 1 gives the
// most chains; NV = 2 halves the chains, and so the workgroups, for
// launches that would otherwise exceed one workgroup per CU (the ring takes
// most of a CU's LDS, so a second workgroup cannot share the CU): each step
// then reads the same A1 / A2 once for twice the columns.
//
// Synchronisation uses the two per-step barriers of the step itself:
// slot p % 3 is read by the compute waves in step p; the loaders refill it
// for step p + 3 after the first barrier (forward launch) or the second
// (backward launches) of step p + 1, and wait for step p + 1's blocks
// before the first barrier of step p + 1.
//
// DEEP (backward launches with NV = 1): four slots, the blocks requested
// three steps ahead instead of two. A step's reads take longer to arrive
// than two steps of compute when every CU streams at once, and the fourth
// slot just fits: 4 x 39,424 B of ring + 6 KiB of exchange = 160 KiB.
template <int NV, bool DEEP = false>
struct Fed {
    static constexpr int A1 = 0;                   // 16 frag tiles of A1
    static constexpr int A2 = 16384;               // 16 frag tiles of A2^T, slots by tr_slot
    static constexpr int C1 = 32768;               // 4 NV ctiles of C1 (value tiles NV vs ..)
    static constexpr int C2 = C1 + NV * 2048;      // 8 NV ctiles of C2 (reverse)
    static constexpr int GN = C2 + NV * 4096;      // gn (512 B)
    static constexpr int SLOT = GN + 512;
    static constexpr int NSLOT = DEEP ? 4 : 3;
    static constexpr int DEPTH = NSLOT - 1;         // steps requested ahead
    static constexpr int NB_FWD = 32 + 2 * NV + 1;  // blocks per step (the last is gn)
    static constexpr int NB_BWD = 32 + 6 * NV + 1;
    static constexpr int XCH = NV * 6;              // LDS exchange: NV x (4 state + 2 Z) slabs
};

// s_waitcnt on the vector-memory counter only (expcnt and lgkmcnt at their
// maxima), and on the LDS counter only.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// Workgroup barrier with no implied waits (each side waits for exactly what
// the other reads after it); the clobber keeps memory accesses in place.
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }

// Loader wave J (0..3): blocks J, J + 4, ... of one step into `slot`. The
// block count is padded to a multiple of four by repeating the gn block
// (same bytes to the same place); a gn block is two copies (fed_loads).
// NOC: no C1 / C2 blocks (a walk of the homogeneous recurrence, which maps
// an entry state to an exit state; see the two-level walks below).
template <bool BWD, int J, int NV, bool DEEP, bool NOC>
__device__ __forceinline__ void fed_issue(const Inter& it, int64_t t, int vs, uint8_t* slot)
{
    using L = Fed<NV, DEEP>;
    constexpr int NB = NOC ? 33 : BWD ? L::NB_BWD : L::NB_FWD;
    constexpr int NPAD = (NB + 3) / 4 * 4;
    // ends of the C1 and C2 blocks
    constexpr int E1 = NOC ? 32 : 32 + 2 * NV, E2 = NOC ? 32 : E1 + 4 * NV;
    const int l = lane_id();
    // A2 is the transpose of the other direction's A1: its frag tiles are
    // copied as they are and read transposed (ld_frag_t64x128)
    const bf16* A1 = BWD ? it.Kt : it.Wn;
    const bf16* A2 = BWD ? it.Wn : it.Kt;
    const bf16* C1 = BWD ? it.X : it.U;
    // The slices of a head read the same A1 / A2 tiles; each starts at a
    // different tile (rotation by 16 / (8 / NV) per slice) so that they do
    // not request the same lines at the same moment.
    const int rot = 2 * NV * vs;
#pragma unroll
    for (int b = J; b < NPAD; b += 4) {
        const void* src;
        int dst;
        if (b < 16) {
            const int bb = (b + rot) & 15;
            src = A1 + t * (CH * DKD) + bb * 512 + l * 8;
            dst = L::A1 + bb * 1024;
        } else if (b < 32) {
            // slots permuted by tr_slot (lane l lands at position l)
            const int bb = (b - 16 + rot) & 15;
            src = A2 + t * (CH * DKD) + bb * 512 + tr_slot(l) * 8;
            dst = L::A2 + bb * 1024;
        } else if (b < E1) {
            src = C1 + t * (CH * DVD) + vs * NV * 1024 + (b - 32) * 512 + l * 8;
            dst = L::C1 + (b - 32) * 1024;
        } else if (BWD && b < E2) {
            src = it.Y + t * (DKD * DVD) + vs * NV * 2048 + (b - E1) * 512 + l * 8;
            dst = L::C2 + (b - E1) * 1024;
        } else {
            // gn, 512 B: two 4-byte-per-lane copies (lane L lands at 4 L)
            const float* gs = it.gn + t * DKD + l;
            __builtin_amdgcn_global_load_lds(gs, (__attribute__((address_space(3))) void*)(slot + L::GN), 4, 0, 0);
            __builtin_amdgcn_global_load_lds(gs + 64, (__attribute__((address_space(3))) void*)(slot + L::GN + 256),
                                             4, 0, 0);
            continue;
        }
        if (b < 32) {
            lds_dma16(src, slot + dst);
        } else {
            // this slice's own C1 / C2 blocks, read by no other workgroup: a
            // streaming load, which leaves the L2 to the shared A1 / A2 tiles
            // (the recompute pair at (1,8192,16): 115 -> 109 us)
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(slot + dst), 16, 0,
                                             CPOL_NT);
        }
    }
}

// Direct-to-LDS copies loader wave J issues per step: one per block, two
// per gn block (the last block and the padding repeats of it).
template <bool BWD, int J, int NV, bool NOC>
constexpr int fed_loads()
{
    constexpr int E = NOC ? 32 : BWD ? 32 + 6 * NV : 32 + 2 * NV;  // blocks before gn
    constexpr int NPAD = (E + 1 + 3) / 4 * 4;
    int n = 0;
    for (int b = J; b < NPAD; b += 4) n += b < E ? 1 : 2;
    return n;
}

template <bool BWD, int J, int NV, bool OUT, typename T, bool NOC>
__device__ __forceinline__ void fed_loader(const Shape& s, const Inter& it, const SeqView& sq, int vs,
                                           uint8_t* ring, bf16x8 (*xs)[64], T* o)
{
    constexpr bool DEEP = NV == 1 && !OUT;
    using L = Fed<NV, DEEP>;
    constexpr int NL = fed_loads<BWD, J, NV, NOC>();
    const int NT = (int)sq.nchunk;  // >= 1
    auto issue = [&](int p) {
        const int pc = p < NT ? p : NT - 1;  // past the end: the last chunk again
        const int c = BWD ? NT - 1 - pc : pc;
        fed_issue<BWD, J, NV, DEEP, NOC>(it, seq_tile(s, sq, c), vs, ring + (p % L::NSLOT) * L::SLOT);
    };
    if constexpr (!OUT) {
        constexpr int D = L::DEPTH;
#pragma unroll
        for (int q = 0; q < D; ++q) issue(q);
        wait_vm<(D - 1) * NL>();  // step 0 has landed
        for (int p = 0; p < NT; ++p) {
            bar();  // first barrier of step p: slot (p + D) % NSLOT is free
            // Step p + D's blocks are requested only after the second barrier:
            // a loader held up issuing them would otherwise hold the compute
            // waves at that barrier (measured ~1.5% slower).
            bar();  // second barrier of step p
            issue(p + D);
            wait_vm<(D - 1) * NL>();  // step p + 1 has landed (younger: steps p + 2 .. p + D)
        }
    } else {
        // Forward with output: this wave also forms output rows 16 J .. 16 J + 15
        // of every chunk, O = Qg S + Hm Z, from the state and Z slabs the compute
        // waves leave in the LDS exchange (S between the step's two barriers, Z
        // after the second). Its Qg / Hm fragments are read two steps ahead into
        // three rotating register sets, each step's just before that step's
        // ring blocks, so that the wait closing a step -- for the next step's
        // ring blocks -- also covers the fragments the next step uses, and no
        // wait ever has to cover younger ring blocks.
        constexpr int NQ = 6;   // Qg / Hm fragment reads per step
        constexpr int NO = NV;  // output row stores per step (one per value tile)
        bf16x8 (*sS)[4][64] = (bf16x8 (*)[4][64])xs;
        bf16x8 (*sZ)[2][64] = (bf16x8 (*)[2][64])(xs + 4 * NV);
        const int l = lane_id(), r = lane_r(), g = lane_g();
        const bf16x8 Ip0 = ident_pi(0);
        struct QH {
            bf16x8 qg[4], hm[2];
        };
        auto ldo = [&](QH& x, int p) {
            const int64_t t = seq_tile(s, sq, p < NT ? p : NT - 1);  // past the end: the last chunk again
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) x.qg[ks] = ld_frag(it.Qg + t * (CH * DKD), J * 4 + ks);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) x.hm[ks] = ld_frag(it.Hm + t * (CH * CH), J * 2 + ks);
        };
        auto step = [&](const QH& cur, QH& ahead, int p) {
            bar();  // first barrier of step p: the state slabs hold S_p; slot (p + 2) % 3 is free
            ldo(ahead, p + 2);
            issue(p + 2);
            f32x4 acc[NV];
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                acc[u] = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc[u] = mfma(cur.qg[ks], sS[u][ks][l], acc[u]);
            }
            wait_lgkm0();  // S read before the compute waves replace it
            bar();         // second barrier of step p: the Z slabs hold Z_p
#pragma unroll
            for (int u = 0; u < NV; ++u)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) acc[u] = mfma(cur.hm[ks], sZ[u][ks][l], acc[u]);
            wait_lgkm0();  // Z read before the compute waves replace it
            // rows: lane (r, g) gets row 16 J + r, values 16 vt + 4 g .. + 3
            const int row = 16 * J + r;
            T* orow = o + (seq_tok0(s, sq, p) + (int64_t)row * s.H) * DVD;
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                const f32x4 x = mfma(pack_pi(acc[u], zero4()), Ip0, zero4());
                float xv[4] = {x[0], x[1], x[2], x[3]};
                if (row < seq_rows(sq, p)) store4_stream(orow + 16 * (NV * vs + u) + 4 * g, xv);
            }
            // step p + 1's ring blocks and fragments have landed: younger than
            // them are this step's fragment reads, ring blocks and stores (the
            // previous step's stores are waited for too, at worst a little early)
            wait_vm<NL + NQ + NO>();
        };
        QH qa, qb, qc;
        ldo(qa, 0);
        issue(0);
        ldo(qb, 1);
        issue(1);
        wait_vm<NL + NQ>();  // step 0's fragments and ring blocks have landed
        int p = 0;
        for (; p + 3 <= NT; p += 3) {
            step(qa, qc, p);
            step(qb, qa, p + 1);
            step(qc, qb, p + 2);
        }
        if (p < NT) step(qa, qc, p);
        if (p + 1 < NT) step(qb, qa, p + 1);
    }
    // no LDS write may still be in flight when the workgroup's LDS is released
    wait_vm<0>();
}

// xs: the LDS exchange, NV x 4 state slabs then NV x 2 Z slabs of 64 x 16 B.
// STORE: write the state before each step and Z (h, R or dh, Rb).
// init: the initial states ([.][128][128], entry bh; null: zero), or with
// ident the identity (columns 16 (NV vs + u) + r of I). fin: where the final
// states go (entry bh; null: nowhere). NOC: the homogeneous recurrence (no
// C1 / C2 terms).
template <bool BWD, int NV, bool STORE, bool DEEP, bool NOC>
__device__ __forceinline__ void fed_compute(const Shape& s, const Inter& it, const float* init, bool ident,
                                            float* fin, const SeqView& sq, int64_t bh, int vs,
                                            const uint8_t* ring, bf16x8 (*xs)[64])
{
    using L = Fed<NV, DEEP>;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id(), r = lane_r(), g = lane_g();
    const int NT = (int)sq.nchunk;  // 0 for an empty sequence: the state passes through
    bf16x8 (*sS)[4][64] = (bf16x8 (*)[4][64])xs;           // [NV][4][64]
    bf16x8 (*sZ)[2][64] = (bf16x8 (*)[2][64])(xs + 4 * NV);  // [NV][2][64]

    bf16* Sout = BWD ? it.dh : it.h;
    bf16* Zout = BWD ? it.Rb : it.R;

    // state: value tile NV vs + u, key rows 32 w + 16 m + 4 g + i, column 16 (NV vs + u) + r
    f32x4 S[NV][2];
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 32 * w + 16 * m + 4 * g + i, col = 16 * (NV * vs + u) + r;
                S[u][m][i] = ident ? (row == col ? 1.f : 0.f) : init ? init[(bh * DKD + row) * DVD + col] : 0.f;
            }

    for (int p = 0; p < NT; ++p) {
        const int c = BWD ? NT - 1 - p : p;
        const int64_t t = seq_tile(s, sq, c);
        const uint8_t* slot = ring + (p % L::NSLOT) * L::SLOT;
        // state before the update (h_c, or dh_c) as ttiles (key tile 2w + m, value tile NV vs + u),
        // the layout in which the local kernel takes it as an MFMA operand:
        // the state frag (M = value, K = keys) times the identity of key
        // half m is the tile's transpose, exact in bf16.
        // The stored states and corrections (like the forward output rows) are
        // streaming stores: only the local kernel reads them, so in the L2
        // they would only evict the A1 / A2 tiles the slices of a head share
        // (128 -> 117 us for the recompute pair at (1,8192,16)).
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            const bf16x8 sfrag = pack_pi(S[u][0], S[u][1]);
            if constexpr (STORE) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    __builtin_nontemporal_store(
                        pack4(mfma(sfrag, ident_pi(m), zero4())),
                        (bf16x4*)ctile_ptr(Sout + t * (DKD * DVD), (NV * vs + u) * 8 + 2 * w + m));
            }
            sS[u][w][l] = sfrag;
        }
        wait_lgkm0();
        bar();
        bf16x8 sf[NV][4], a1[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            a1[ks] = *(const bf16x8*)(slot + L::A1 + (w * 4 + ks) * 1024 + l * 16);
#pragma unroll
            for (int u = 0; u < NV; ++u) sf[u][ks] = sS[u][ks][l];
        }
        // Z = C1 + A1 S   (rows 16w .. 16w + 15)
        bf16x4 z4[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u) {
            f32x4 z = NOC ? zero4() : unpack4(*(const bf16x4*)(slot + L::C1 + ((u * 4 + w) * 64 + l) * 8));
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) z = mfma(a1[ks], sf[u][ks], z);
            z4[u] = pack4(z);
            *(bf16x4*)((bf16*)&sZ[u][w >> 1][l] + 4 * (w & 1)) = z4[u];
        }
        wait_lgkm0();
        bar();
        if constexpr (STORE) {
            // Rb as the ctile it is; R as a ttile (its transpose by the
            // identity, exact), the layout in which the local kernel takes it
            // as an MFMA operand
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                const bf16x4 zs = BWD ? z4[u] : pack4(mfma(cat8(z4[u], bf16x4{}), ident_pi(0), zero4()));
                __builtin_nontemporal_store(zs, (bf16x4*)ctile_ptr(Zout + t * (CH * DVD), (NV * vs + u) * 4 + w));
            }
        }
        bf16x8 zf[NV][2], a2[2][2];
#pragma unroll
        for (int u = 0; u < NV; ++u)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) zf[u][ks] = sZ[u][ks][l];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) a2[m][ks] = ld_frag_t64x128(slot + L::A2, 2 * w + m, ks);
        // S <- gn S (+ C2) + A2 Z
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const float4 gv = *(const float4*)(slot + L::GN + (32 * w + 16 * m + 4 * g) * 4);
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                f32x4 acc = {gv.x * S[u][m][0], gv.y * S[u][m][1], gv.z * S[u][m][2], gv.w * S[u][m][3]};
                if (BWD && !NOC) {
                    const f32x4 y =
                        unpack4(*(const bf16x4*)(slot + L::C2 + ((u * 8 + 2 * w + m) * 64 + l) * 8));
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] += y[i];
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) acc = mfma(a2[m][ks], zf[u][ks], acc);
                S[u][m] = acc;
            }
        }
    }
    if (fin) {
#pragma unroll
        for (int u = 0; u < NV; ++u)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fin[(bh * DKD + 32 * w + 16 * m + 4 * g + i) * DVD + 16 * (NV * vs + u) + r] = S[u][m][i];
    }
}

template <bool BWD, int NV, bool OUT, typename T, bool STORE, bool NOC = false>
__device__ __forceinline__ void fed_body(const Shape& s, const Inter& it, const SeqView& sq, const float* init,
                                         bool ident, float* fin, int64_t bh, int vs, uint8_t* ring,
                                         bf16x8 (*xs)[64], T* o)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (sq.nchunk <= 0 && w >= 4) return;  // an empty sequence: no steps, no barriers
    switch (w) {
    case 4: fed_loader<BWD, 0, NV, OUT, T, NOC>(s, it, sq, vs, ring, xs, o); break;
    case 5: fed_loader<BWD, 1, NV, OUT, T, NOC>(s, it, sq, vs, ring, xs, o); break;
    case 6: fed_loader<BWD, 2, NV, OUT, T, NOC>(s, it, sq, vs, ring, xs, o); break;
    case 7: fed_loader<BWD, 3, NV, OUT, T, NOC>(s, it, sq, vs, ring, xs, o); break;
    default:
        fed_compute<BWD, NV, STORE, NV == 1 && !OUT, NOC>(s, it, init, ident, fin, sq, bh, vs, ring, xs);
        break;
    }
}

// ---------------------------------------------------------------------------
// Two-level walks. With few walks (small B * H) a serial walk over every
// chunk leaves most CUs idle, while its step time is bound by latency. The
// state recurrence is affine in the state: a walk over chunks [a, b) maps
// its entry state S to Phi S + E, with Phi the product of the homogeneous
// steps (the forward walk's S <- diag(gn) S - Kt^T W S, the reverse walk's
// transpose) and E the exit state from S = 0 (ReWY paper Sec. 2.1: the
// scan is serial across chunks; the chunk-affine composition of such maps
// is the two-level form). The walk is cut into segments:
//   1. for every segment but the last in walk order, Phi (the walk from the
//      identity without the C terms) and E (the walk from zero), all
//      segments at once (scan_sum_kernel);
//   2. the entry state of every segment by S <- Phi S + E through the
//      segments in walk order, in fp32 (scan_combine_kernel);
//   3. every segment's own walk from its entry state, storing what the
//      one-level walk stores (scan_fed_kernel with it.nseg segments).
// Steps 1 and 3 each take a segment's length in serial steps instead of the
// whole walk's.

// Chunks of segment sg of a walk over nchunk chunks.
__device__ __forceinline__ SeqView segment_of(const Inter& it, const SeqView& sq, int sg)
{
    const int64_t c0 = sg * it.seglen, left = sq.nchunk - c0;
    return seg_view(sq, c0, left < it.seglen ? (left > 0 ? left : 0) : it.seglen);
}

// One chain of a walk launch: its segment (two-level walks), where its
// initial state comes from and where its final state goes.
template <bool BWD, int NV, bool OUT, typename T, bool STORE>
__device__ __forceinline__ void walk_chain(const Shape& s, const Inputs& in, const Inter& it, float* fin,
                                           const Chain& ch, uint8_t* ring, bf16x8 (*xs)[64], T* o)
{
    SeqView sq = seq_view(s, ch.n, ch.hd);
    const float* init = BWD ? in.dht : in.h0;
    if (it.nseg > 1) {
        sq = segment_of(it, sq, ch.sg);
        const bool first = BWD ? ch.sg == it.nseg - 1 : ch.sg == 0;
        const bool last = BWD ? ch.sg == 0 : ch.sg == it.nseg - 1;
        if (!first) init = it.seg_ent + ((int64_t)(BWD ? 1 : 0) * it.nseg + ch.sg) * s.NS * s.H * (DKD * DVD);
        if (!last) fin = nullptr;
    }
    fed_body<BWD, NV, OUT, T, STORE>(s, it, sq, init, false, fin, ch.n * s.H + ch.hd, ch.vs, ring, xs, o);
}

// Backward launches (OUT = false): ndir = 2 runs forward and reverse chains
// side by side (the reverse scan reads only prep's operands, not the
// forward states); ndir = 1 the reverse scan alone. Only the reverse chains
// write fin (dh0). The forward launch (OUT = true, ndir = 1) writes the
// output o and fin (ht), and h and R when STORE (full save). With
// it.nseg > 1 each chain walks one segment (step 3 above).
template <int NV, bool OUT, typename T, bool STORE>
__global__ __launch_bounds__(512) void scan_fed_kernel(Shape s, Inputs in, Inter it, float* fin, int ndir, T* o)
{
    using L = Fed<NV, NV == 1 && !OUT>;
    __shared__ __attribute__((aligned(16))) uint8_t ring[L::NSLOT * L::SLOT];
    __shared__ bf16x8 xs[L::XCH][64];
    Chain ch;
    if (!chain_of_block(s, NVS / NV, ndir, !OUT, blockIdx.x, ch, it.nseg)) return;
    if constexpr (OUT) {
        walk_chain<false, NV, true, T, STORE>(s, in, it, fin, ch, ring, xs, o);
    } else {
        if (ch.bwd) walk_chain<true, NV, false, T, STORE>(s, in, it, fin, ch, ring, xs, o);
        else walk_chain<false, NV, false, T, STORE>(s, in, it, nullptr, ch, ring, xs, o);
    }
}

// Step 1: chains (walk, summarized segment, slice vs < 16). Slices 0..7
// walk the homogeneous recurrence from columns 16 vs .. 16 vs + 15 of the
// identity (Phi), slices 8..15 the full recurrence from zero (E, value
// columns 16 (vs - 8) ..). The forward walk summarizes segments
// 0 .. nseg - 2, the reverse walk 1 .. nseg - 1 (its last in walk order is
// segment 0); a segment's summary sits at its position among those.
__global__ __launch_bounds__(512) void scan_sum_kernel(Shape s, Inter it, int ndir, int bwd1)
{
    using L = Fed<1, true>;
    __shared__ __attribute__((aligned(16))) uint8_t ring[L::NSLOT * L::SLOT];
    __shared__ bf16x8 xs[L::XCH][64];
    Chain ch;
    if (!chain_of_block(s, 2 * NVS, ndir, bwd1 != 0, blockIdx.x, ch, it.nseg - 1)) return;
    const SeqView sq = segment_of(it, seq_view(s, ch.n, ch.hd), ch.bwd ? ch.sg + 1 : ch.sg);
    const bool phi = ch.vs < NVS;
    const int vs = ch.vs & (NVS - 1);
    float* fin = it.seg_sum + (((int64_t)(ch.bwd ? 1 : 0) * (it.nseg - 1) + ch.sg) * s.NS * s.H +
                               ch.n * s.H + ch.hd) * 2 * (DKD * DVD) + (phi ? 0 : DKD * DVD);
    bf16* const no = nullptr;
    if (ch.bwd) {
        if (phi) fed_body<true, 1, false, bf16, false, true>(s, it, sq, nullptr, true, fin, 0, vs, ring, xs, no);
        else fed_body<true, 1, false, bf16, false, false>(s, it, sq, nullptr, false, fin, 0, vs, ring, xs, no);
    } else {
        if (phi) fed_body<false, 1, false, bf16, false, true>(s, it, sq, nullptr, true, fin, 0, vs, ring, xs, no);
        else fed_body<false, 1, false, bf16, false, false>(s, it, sq, nullptr, false, fin, 0, vs, ring, xs, no);
    }
}

// Step 2: one workgroup per (state entry bh, direction, 16 value columns).
// A segment's Phi (64 KiB) goes to LDS, read from global memory a segment
// ahead into registers; S <- Phi S + E runs on the fp32 MFMA (wave w: state
// rows 32 w .. 32 w + 31, all 16 columns), so the chained entry states are
// exact fp32 products.
__global__ __launch_bounds__(256) void scan_combine_kernel(Shape s, Inputs in, Inter it, int ndir, int bwd1)
{
    const int64_t bh = blockIdx.x, NSH = s.NS * s.H;
    const bool bwd = ndir == 2 ? blockIdx.y == 1 : bwd1 != 0;
    const int64_t d = bwd ? 1 : 0;
    const int c0 = 16 * blockIdx.z;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
    __shared__ float S[DKD][16];
    __shared__ __attribute__((aligned(16))) float P[DKD][DKD + 4];  // padded rows: conflict-free operand reads
    const float* init = bwd ? in.dht : in.h0;
    {
        const int row = tid >> 1, cb = (tid & 1) * 8;
#pragma unroll
        for (int j = 0; j < 8; ++j) S[row][cb + j] = init ? init[(bh * DKD + row) * DVD + c0 + cb + j] : 0.f;
    }
    const int nseg = it.nseg;
    // the k-th segment summarized in walk order: its Phi and E
    auto summary = [&](int k) -> const float* {
        const int cur = bwd ? nseg - 1 - k : k;
        const int pos = bwd ? cur - 1 : cur;  // its position among the summarized segments
        return it.seg_sum + ((d * (nseg - 1) + pos) * NSH + bh) * 2 * (DKD * DVD);
    };
    float4 pv[16];
    auto load_phi = [&](int k) {
        const float* phi = summary(k);
#pragma unroll
        for (int u = 0; u < 16; ++u) pv[u] = *(const float4*)(phi + (u * 256 + tid) * 4);
    };
    if (nseg > 1) load_phi(0);
    for (int k = 0; k + 1 < nseg; ++k) {
        const int cur = bwd ? nseg - 1 - k : k, nxt = bwd ? cur - 1 : cur + 1;
        const float* E = summary(k) + DKD * DVD;
        // accumulators start from E: lane (r, g) element i is row 16 mt + 4 g + i, column r.
        // (E is read before the next Phi is requested: loads complete in
        // order, so the wait for E then does not wait for that Phi.)
        f32x4 acc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[m][i] = E[(32 * w + 16 * m + 4 * g + i) * DVD + c0 + r];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int e = (u * 256 + tid) * 4;
            *(float4*)&P[e / DKD][e % DKD] = pv[u];
        }
        if (k + 2 < nseg) load_phi(k + 1);  // the next segment's Phi, while this one runs
        __syncthreads();  // P and S complete
#pragma unroll 8
        for (int ks = 0; ks < DKD / 4; ++ks) {
            const float b = S[4 * ks + g][r];
#pragma unroll
            for (int m = 0; m < 2; ++m) acc[m] = mfma4(P[32 * w + 16 * m + r][4 * ks + g], b, acc[m]);
        }
        __syncthreads();  // every read of S and P is done
        float* ent = it.seg_ent + ((d * nseg + nxt) * NSH + bh) * (DKD * DVD);
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 32 * w + 16 * m + 4 * g + i;
                S[row][r] = acc[m][i];
                ent[row * DVD + c0 + r] = acc[m][i];
            }
    }
}

}  // namespace

int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

namespace {

// One workgroup per CU fits (LDS); NV = 2 when NV = 1 would need more than
// one round of workgroups.
bool wide(const Shape& s, int ndir, int nseg) { return s.NS * s.H * NVS * ndir * nseg > cu_count(); }

// Steps 1 and 2 of the two-level walks (a no-op for one-level walks).
hipError_t two_level_prefix(const Shape& s, const Inputs& in, const Inter& it, int ndir, bool bwd1,
                            hipStream_t st)
{
    if (it.nseg <= 1) return hipSuccess;
    scan_sum_kernel<<<scan_grid(s, 2 * NVS, ndir, it.nseg - 1), 512, 0, st>>>(s, it, ndir, bwd1 ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    scan_combine_kernel<<<dim3((unsigned)(s.NS * s.H), (unsigned)ndir, NVS), 256, 0, st>>>(s, in, it, ndir,
                                                                                       bwd1 ? 1 : 0);
    return hipGetLastError();
}

// The walk launches' view of it: at least one segment.
Inter walk_args(const Inter& it)
{
    Inter jt = it;
    if (jt.nseg < 1 || !jt.seg_sum || !jt.seg_ent) jt.nseg = 1;
    return jt;
}

hipError_t launch_fed(const Shape& s, const Inputs& in, const Inter& it0, float* dh0, int ndir,
                      hipStream_t st)
{
    const Inter it = walk_args(it0);
    hipError_t e = two_level_prefix(s, in, it, ndir, true, st);
    if (e != hipSuccess) return e;
    const int ns = it.nseg;
    if (wide(s, ndir, ns))
        scan_fed_kernel<2, false, bf16, true><<<scan_grid(s, NVS / 2, ndir, ns), 512, 0, st>>>(s, in, it, dh0, ndir,
                                                                                             nullptr);
    else
        scan_fed_kernel<1, false, bf16, true><<<scan_grid(s, NVS, ndir, ns), 512, 0, st>>>(s, in, it, dh0, ndir,
                                                                                         nullptr);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fed_out(const Shape& s, const Inputs& in, const Inter& it0, T* o, float* ht, hipStream_t st)
{
    const Inter it = walk_args(it0);
    hipError_t e = two_level_prefix(s, in, it, 1, false, st);
    if (e != hipSuccess) return e;
    const int ns = it.nseg;
    const unsigned g2 = scan_grid(s, NVS / 2, 1, ns), g1 = scan_grid(s, NVS, 1, ns);
    if (it.h) {  // full save: h and R too
        if (wide(s, 1, ns)) scan_fed_kernel<2, true, T, true><<<g2, 512, 0, st>>>(s, in, it, ht, 1, o);
        else scan_fed_kernel<1, true, T, true><<<g1, 512, 0, st>>>(s, in, it, ht, 1, o);
    } else {
        if (wide(s, 1, ns)) scan_fed_kernel<2, true, T, false><<<g2, 512, 0, st>>>(s, in, it, ht, 1, o);
        else scan_fed_kernel<1, true, T, false><<<g1, 512, 0, st>>>(s, in, it, ht, 1, o);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_fwd(const Shape& s, const Inputs& in, const Inter& it, void* o, float* ht,
                           hipStream_t st)
{
    if (!o) return hipErrorInvalidValue;
    return s.f32 ? launch_fed_out(s, in, it, (float*)o, ht, st) : launch_fed_out(s, in, it, (bf16*)o, ht, st);
}

hipError_t launch_scan_bwd(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                           hipStream_t st)
{
    return launch_fed(s, in, it, dh0, 1, st);
}

hipError_t launch_scan_pair(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                            hipStream_t st)
{
    return launch_fed(s, in, it, dh0, 2, st);
}

}  // namespace gdr
