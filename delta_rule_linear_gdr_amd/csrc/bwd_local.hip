// Chunk-local backward of the chunkwise gated delta rule, one workgroup per
// (chunk, head), after the reverse state scan has produced Rb (the summed
// correction adjoint) and dh (the adjoint of the state at the chunk end).
//
// Producer (ReWY paper, paperpeel.com/paper/2611.01940, Sec. 3.1, and the
// onedev.kr summary, "How it works"):
//   P = A^T Rb;  dv = beta * P;  D = -strict_lower(P R^T);  Eb_dir = -P h^T
// Output coefficient adjoint: Hb = lower_incl(dO R^T).
// State-direct terms: Qgb = dO h^T, Ktb = R dh^T (paper Sec. 3.5: the joint
// consumer takes the sensitivity and state-direct terms together).
// Consumers of D and Hb:
//   scalar gate -- Gram elimination (Sec. 3.4; onedev.kr "What is different"):
//     Gam = D o Lam, Gq = Hb o Lam, Lam_ij = exp(G_i - G_j);
//     A_K = Gam K, B_K = Gam^T diag(beta) K, Gq K, Gq^T Q;
//     dk += beta A_K + B_K + Gq^T Q,  dq += Gq K,  dbeta += <k, A_K>,
//     Gbar += beta <k, A_K> - <k, B_K> + <q, Gq K> - <k, Gq^T Q>
//   vector gate -- centred matrix intra (Sec. 3.3, "Centered factors"):
//     alpha = exp(G - c), zeta = exp(c - G);
//     U_q = Hb Y', U_e = D Y', U_y = Hb^T Q' + D^T E'  (Y' = zeta K,
//     Q' = alpha Q, E' = beta alpha K);
//     dq += alpha U_q, dk += beta alpha U_e + zeta U_y,
//     dbeta += <U_e, alpha k>, Gbar += Q' U_q + E' U_e - Y' U_y
//     applied per 16-token window (one token tile): the products within a
//     window use its centre c = (max G + min G)/2; every block of a row
//     tile m against another window's columns uses a boundary pivot (G at
//     token 16 m - 1 for the earlier windows, in Hb Y' and D Y'; G at token
//     16 m + 16 for the later ones, in Hb^T Q' and D^T E'), so that both of
//     its factors are at most 1 for decays g <= 0. The factors then span
//     exp(+-range of 16 tokens / 2) rather than that of the chunk, which
//     keeps strong decays within fp32 range. A 32-token contraction slab
//     that holds two windows with different factors is split into its two
//     16-token halves (K = 16 products).
// Feature-local chain rules for the remaining terms, with gam = exp(G):
//   dq += gam Qgb;  dk += beta gam Eb_dir + exp(G_n - G) Ktb;
//   dbeta += <P, v> + <Eb_dir, gam k>   (undivided form, App. B.3)
//   Gbar += gam q Qgb + beta gam k Eb_dir - exp(G_n - G) k Ktb;
//   Gbar_n += sum_j exp(G_n - G_j) k_j Ktb_j + gam_n rowsum(h o dh)
// and dg is the chunk-local reverse cumsum of Gbar (Sec. 3.5), summed over
// features for a scalar gate (App. E.1).
// GDN2 (paper Table 1; its erase and write gradients stay separate, Sec. 3.1):
// the vector-gate kernel with E = ers o gam o K and Z = wrt o V, so every
// beta of the erase path becomes the per-(token, key) erase gate, dv = wrt o P,
// and the gate gradients are written entry by entry instead of summed:
// dwrt = v o P, ders = gam k o (Eb_dir + Eb_intra) (= the per-feature terms
// the beta gradient would sum).
//
// Schedule (eight waves; wave w owns feature tile [16 w, 16 w + 16) of
// every 64 x 128 product, all 64 token rows, so the chain rules and the
// gradient accumulators stay in that wave's registers):
//   1. P^T = Rb^T A from the Rb accumulator tiles (no transpose needed);
//      dv and <P, v> from it; P, R, dO fragments (contraction over values)
//      into LDS; h, dh fragments (read as stored: the scans write them as
//      ttiles, whose lane pieces pair up into frag slabs) and the rowsum
//      of h o dh in registers;
//      K, Q in accumulator order through K * I (exact).
//   2. D and Hb tiles (contraction over values) into LDS as the A operands
//      of the Gram / matrix-intra products, D^T and Hb^T read from the same
//      tiles with gfx950's transposing LDS read; Eb_dir, Qgb, Ktb.
//   3. The four consumer products; reductions of dbeta and dg.
// Orientation changes use MFMA products with the identity, which are exact.
//
// Launch: the scalar-gate three-product kernel is persistent (one workgroup
// per CU, each taking every G-th (chunk, head)) and streams the next
// chunk's h and dh into LDS while it works on the current one; the
// vector-gate and seven-product kernels, which have no LDS left for that,
// run one workgroup per (chunk, head).
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int NW = 8;
constexpr int NTHR = 64 * NW;

__device__ __forceinline__ void st_half(bf16x8* buf, int tile, int half, const bf16x4& v)
{
    *(bf16x4*)((bf16*)&buf[tile * 64 + lane_id()] + 4 * half) = v;
}
// The same into a buffer whose slots are placed by tr_slot (read plainly at
// tr_slot(lane), or transposed by ld_frag_t64x64).
__device__ __forceinline__ void st_half_tr(bf16x8* buf, int tile, int half, const bf16x4& v)
{
    *(bf16x4*)((bf16*)&buf[tile * 64 + tr_slot(lane_id())] + 4 * half) = v;
}

// Prefetch of h and dh (persistent form): wave w copies the sixteen
// fragments it reads itself -- ttiles vt * 8 + w (vt = 0..7) of h, then of
// dh, 512 bytes each -- into its own 8 KiB staging area, two tiles per
// 16-byte-per-lane direct-to-LDS load. A tile is copied verbatim, so lane
// l's four elements of tile vt land at entry vt * 64 + l (h) and
// 512 + vt * 64 + l (dh) of the area.
//
// The loads are issued from inline assembly, which the compiler's wait
// insertion does not see: it would otherwise make later LDS writes of the
// chunk wait for them (it cannot tell the staging area from the other LDS
// buffers) and so serialize the prefetch. Their completion is awaited
// explicitly instead (PF_WAIT below). Untracked loads issued after a
// tracked one only make the compiler's own counts conservative, since
// vector-memory operations complete in order.
constexpr int STAGE = 1024;  // bf16x4 entries per wave

__device__ __forceinline__ void dma16_untracked(const bf16* src, uint32_t lds_addr)
{
    // the LDS base goes in M0 (set by the compiler just before); one wait
    // state between writing M0 and the load
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ void stage_hdh(const Inter& it, int64_t tt, int w, bf16x4* area)
{
    const int l = lane_id();
    const bf16* const hs = it.h + tt * (DKD * DVD);
    const bf16* const ds = it.dh + tt * (DKD * DVD);
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16x4*)area);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int off = ((2 * j + (l >> 5)) * 8 + w) * 256 + (l & 31) * 8;
        dma16_untracked(hs + off, base + j * 1024);
        dma16_untracked(ds + off, base + 4096 + j * 1024);
    }
}

// Where a chunk reads its staged h and dh (phase 1c), at least the 32 reads
// of the chunk's own batch have been issued after the staging loads (which
// were issued during the previous chunk, or before the first), so
// vmcnt(PF_WAIT) with PF_WAIT < 32 leaves none of them outstanding.
constexpr int PF_WAIT = 8;

// The last phase of a chunk (the dbeta and dg reductions over the eight
// waves' partials) as the persistent form defers it: run by the next chunk
// once its reads are issued, so that it overlaps their latency.
template <typename T>
struct Tail {
    T* dbo;
    float* dgo;
    int nv;
    bool on;
};

// One (chunk, head). PF: h and dh come from this wave's staging area
// `area` (already requested), and the next chunk's (tile tnext >= 0) are
// requested once they have been read; the previous chunk's deferred last
// phase (*pend) runs after this chunk's reads are issued, and this chunk's
// is left in *pend when a next chunk follows.
template <typename T, bool VEC, bool WY7, bool PF, bool GD2>
__device__ __forceinline__ void bwd_local_chunk(const Shape& s, const Inputs& in, const Inter& it,
                                                const Grads& gr, const ChunkRef& cr,
                                                int64_t tnext, bf16x4* area, Tail<T>* pend)
{
    const int64_t t = cr.t;
    const int64_t tok0 = cr.tok0;  // token row of the chunk's row 0
    const int nv = cr.nv;          // rows past it read as zeros and are not written
    // Row stride (elements) of q, k, v, dO and their gradients. In-chunk
    // offsets stay below 64 * H * 128 < 2^31 (H <= 65535), so they are 32-bit
    // and every pointer below is a uniform per-chunk base.
    const int ld = (int)(s.H * DKD);
    const int Hs = (int)s.H;
    const int tid = threadIdx.x;
    // The lane index, opaque to the compiler in the persistent form:
    // lane-only values (the identity fragments, lane offsets) are then
    // formed per chunk instead of being hoisted out of the loop and held in
    // registers across it.
    int lx = lane_id();
    if (PF) asm volatile("" : "+v"(lx));
    const int l = lx, r = lx & 15, g = (lx >> 4) & 3;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int f = 16 * w + r;  // this lane's feature (key or value) column

    // LDS fragment buffers (16 x 32 frag tiles; 1024 entries = 64 x 128,
    // 512 entries = 64 x 64). Both producers: R, dO (M = tok, K = val) and the
    // consumer A operands GT, GqT (and Gm, Gq: TRG below). ReWY: P (M = tok,
    // K = val). The
    // seven-product producer: Rb, Z (M = tok, K = val), E, W (M = tok,
    // K = key) with W = Rb h^T, Abar^T (M = col, K = row) and X (M = tok,
    // K = tok) with X = A^T Abar.
    // Vector gate (ReWY): each wave also parks the lo halves of its centred
    // consumer operands (3 operands x 2 token slabs) at lds + NLDS + w * 384;
    // the seven-product variant has no LDS left for them and keeps them in
    // registers.
    constexpr bool LO_LDS = VEC && !WY7;
    // TRG: D and Hb stored once, D^T and Hb^T read from them transposed
    // (see lGT below); the vector-gate seven-product kernel keeps all four
    constexpr bool TRG = !(VEC && WY7);
    constexpr int NLDS = WY7 ? (TRG ? 8192 : 9216) : 4096;
    __shared__ bf16x8 lds[NLDS + (LO_LDS ? NW * 6 * 64 : 0)];
    bf16x8* const lLo = lds + NLDS + (LO_LDS ? w * 6 * 64 : 0);
    bf16x8 loReg[LO_LDS ? 1 : 6];
    auto lo_get = [&](int x) -> bf16x8 { return LO_LDS ? lLo[x * 64 + l] : loReg[LO_LDS ? 0 : x]; };
    auto lo_set = [&](int x, const bf16x8& v) {
        if (LO_LDS) lLo[x * 64 + l] = v;
        else loReg[LO_LDS ? 0 : x] = v;
    };
    bf16x8* const lR = lds;
    bf16x8* const lO = lds + 1024;
    bf16x8* const lP = lds + 2048;                      // ReWY
    bf16x8* const lRb = lds + 2048;                     // seven-product
    bf16x8* const lZ = lds + 3072;
    bf16x8* const lE = lds + 4096;
    bf16x8* const lWb = lds + 5120;
    bf16x8* const lAbT = lds + 6144;
    bf16x8* const lX = lds + 6656;
    bf16x8* const lG = lds + (WY7 ? 7168 : 3072);
    // TRG: D and Hb only, slots placed by tr_slot, D^T and Hb^T read from
    // them with transposing LDS reads; otherwise all four, plainly
    bf16x8* const lGm = lG;
    bf16x8* const lGT = lG + (TRG ? 0 : 512);
    bf16x8* const lGq = lG + 1024;
    bf16x8* const lGqT = lG + (TRG ? 512 : 1536);
    __shared__ __attribute__((aligned(16))) float sG[CH], sBeta[CH];
    // per-token partial sums of the eight waves (token-major: a token's eight
    // partials are two 16-byte reads)
    __shared__ __attribute__((aligned(16))) float sRedB[CH][NW], sRedP[CH][NW], sRedG[CH][NW];
    __shared__ float sExtra[DKD];
    // scalar gate: exp(G) and exp(G_n - G) per token (wave 0, with the gate scan)
    __shared__ __attribute__((aligned(16))) float sGam[VEC ? 4 : CH], sKt[VEC ? 4 : CH];
    __shared__ __attribute__((aligned(16))) float sEx[NW];
    // GDN2: the chunk's erase gates (token rows, per key), rows padded by 16
    // bytes so that the four row groups of a read fall on different banks
    constexpr int EST = DKD + 8;
    __shared__ __attribute__((aligned(16))) bf16 sErs[GD2 ? CH * EST : 8];

    const T* q = (const T*)in.q + tok0 * DKD;
    const T* k = (const T*)in.k + tok0 * DKD;
    const T* v = (const T*)in.v + tok0 * DVD;
    const T* dO = (const T*)in.dO + tok0 * DVD;
    const float* gin = in.g + (VEC ? tok0 * DKD : tok0);
    T* dqo = (T*)gr.dq + tok0 * DKD;
    T* dko = (T*)gr.dk + tok0 * DKD;
    T* dvo = (T*)gr.dv + tok0 * DVD;
    float* dgo = gr.dg + (VEC ? tok0 * DKD : tok0);
    const T* betai = (const T*)in.beta + tok0;
    T* dbo = (T*)gr.dbeta + tok0;

    // ---- every global read of this chunk, issued before the first is used
    //      (one memory round trip instead of one per phase) ----
    // Persistent form (bf16): the chunk's v, dO, k, q rows (4 x 64 x 128)
    // are first copied into the front 64 KiB of the fragment buffers, which
    // phase 1 is the first to write, with coalesced direct-to-LDS loads
    // (1 KiB = four whole rows per instruction). Each wave then reads its
    // 16-column slices from there.
    // Read from global memory, a slice takes 8 bytes of 16 rows per
    // instruction: 16 cache lines of which it uses a quarter, every line
    // fetched by four waves. A row's 16-byte chunk j is stored at j ^ (row &
    // 15), so that the 16 rows of a slice read fall on distinct banks.
    // (bwd_local at (1,8192,16): 141 -> 137 us. The per-chunk kernels, the
    // vector-gate one in particular, lost more to the extra barrier and the
    // earlier wait than they gained, so they read their slices directly.)
    constexpr bool SROW = sizeof(T) == 2 && PF;
    bf16* const stg = (bf16*)lds;
    if constexpr (SROW) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = w * 8 + i, mat = j >> 4, row = 4 * (j & 15) + (l >> 4);
            const int rcl = row < nv ? row : nv - 1;  // rows past nv: row nv - 1 (masked where read)
            const T* src = mat == 0 ? v : mat == 1 ? dO : mat == 2 ? k : q;
            lds_dma16(src + rcl * ld + ((l & 15) ^ (row & 15)) * 8, stg + (mat * CH + 4 * (j & 15)) * DKD);
        }
    }
    typedef decltype(ld4raw(q)) R4;
    typedef decltype(ld8raw(q)) R8;
    const bf16* const Rbg = it.Rb + t * (CH * DVD);
    const bf16* const Rg = it.R + t * (CH * DVD);
    const bf16* const hg = it.h + t * (DKD * DVD);
    const bf16* const dhg = it.dh + t * (DKD * DVD);
    const bf16* const ATg = it.AT + t * (CH * CH);
    const bf16* const Afg = it.Af + t * (CH * CH);
    // (beta and a scalar gate are read by every wave, so that no branch
    // has to wait for them)
    // Rows past nv: the read is made from a clamped row (always in range, so
    // it stays an unconditional read in the batch) and its value replaced by
    // zero with a select.
    const int lc = l < nv ? l : nv - 1;
    const T bload = GD2 ? (T)0.f : betai[lc * Hs];
    const T braw = l < nv ? bload : (T)0.f;
    float graw[VEC ? 16 : 1];
    if (VEC) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e)
            {
                const int i = 16 * m + 4 * g + e;
                const float gl = gin[(i < nv ? i : nv - 1) * ld + f];
                graw[VEC ? 4 * m + e : 0] = i < nv ? gl : 0.f;
            }
    } else {
        const float gl = gin[lc * Hs];
        graw[0] = l < nv ? gl : 0.f;
    }
    bf16x4 rbq[4], rq[4], hq[8], dhq[8];
    bf16x8 atf[6];  // A^T frags m * 2 + 1 (m = 0..3), then m * 2 + 0 (m = 0, 1)
    // Every wave multiplies by all six nonzero A^T frags. The persistent form
    // copies them once into LDS (wave j < 6 copies frag j of atf's order) and
    // each wave reads them from there after the first barrier, instead of
    // eight waves fetching the same 6 KiB (bwd_local at (1,8192,16): 136.7
    // -> 135.4 us).
    __shared__ bf16x8 sAT[SROW ? 6 * 64 : 1];
    R4 vr[4], orw[4];
    R4 kr[4], qr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rbq[i] = *(const bf16x4*)ctile_ptr(Rbg, w * 4 + i);
    if constexpr (SROW) {
        if (w < 6) lds_dma16(frag_ptr(ATg, w < 4 ? w * 2 + 1 : (w - 4) * 2), sAT + w * 64);
    } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) atf[m] = ld_frag(ATg, m * 2 + 1);
        atf[4] = ld_frag(ATg, 0);
        atf[5] = ld_frag(ATg, 2);
    }
    // token row 16 m + r, clamped into the chunk (zeros past nv)
    auto rowc = [&](int m) { return 16 * m + r < nv ? 16 * m + r : nv - 1; };
    const bool rv[4] = {r < nv, 16 + r < nv, 32 + r < nv, 48 + r < nv};
    if constexpr (!SROW) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const R4 x = ld4raw(v + rowc(m) * ld + 16 * w + 4 * g);
            vr[m] = rv[m] ? x : R4{};
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) rq[i] = *(const bf16x4*)ctile_ptr(Rg, w * 4 + i);
    if constexpr (!SROW) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const R4 x = ld4raw(dO + rowc(m) * ld + 16 * w + 4 * g);
            orw[m] = rv[m] ? x : R4{};
        }
    }
    if (!PF) {
#pragma unroll
        for (int vt = 0; vt < 8; ++vt) {
            hq[vt] = *(const bf16x4*)ctile_ptr(hg, vt * 8 + w);
            dhq[vt] = *(const bf16x4*)ctile_ptr(dhg, vt * 8 + w);
        }
    }
    if constexpr (!SROW) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // this wave's 16 keys only (as for v): lane (r, g) gets keys 16 w + 4 g .. + 3
            const R4 xk = ld4raw(k + rowc(m) * ld + 16 * w + 4 * g);
            const R4 xq = ld4raw(q + rowc(m) * ld + 16 * w + 4 * g);
            kr[m] = rv[m] ? xk : R4{};
            qr[m] = rv[m] ? xq : R4{};
        }
    }
    // GDN2: the erase gates of the chunk (two 16-byte row pieces per thread,
    // for LDS) and the write gates of this lane's P entries
    bf16x8 eraw[GD2 ? 2 : 1];
    bf16x4 wraw[GD2 ? 4 : 1];
    if constexpr (GD2) {
        const bf16* ers = (const bf16*)in.ers + tok0 * DKD;
        const bf16* wrt = (const bf16*)in.wrt + tok0 * DVD;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int id = tid + NTHR * u, i = id >> 4, c = (id & 15) * 8;
            const bf16x8 x = *(const bf16x8*)(ers + (i < nv ? i : nv - 1) * ld + c);
            eraw[u] = i < nv ? x : bf16x8{};
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const bf16x4 x = *(const bf16x4*)(wrt + rowc(m) * ld + 16 * w + 4 * g);
            wraw[m] = rv[m] ? x : bf16x4{};
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. (defined here, run last or deferred) dbeta (wave 1); scalar
    //      gate: dg (wave 0), side by side, from the partials in LDS ----
    auto sum8 = [](const float* p) {
        const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
        return ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
    };
    auto last_phase = [&](T* dbo_, float* dgo_, int nv_) {
        if (!GD2 && w == 1) {
            const float sb = sum8(sRedB[l]) + sum8(sRedP[l]);
            if (l < nv_) io<T>::st(dbo_ + l * Hs, sb);
        }
        if (!VEC && w == 0) {
            // sum the extra over features, then reverse cumsum over tokens
            float xg = sum8(sRedG[l]);
            if (l == CH - 1) xg += sum8(sEx);
            xg = wave_incl_suffix(xg);
            if (l < nv_) dgo_[l * Hs] = xg;
        }
    };
    if (PF && pend->on) {
        // the previous chunk's: its partials stay untouched until this
        // chunk's first barrier, which waves 0 and 1 reach only afterwards
        last_phase(pend->dbo, pend->dgo, pend->nv);
        pend->on = false;
    }

    // ---- 0. gates, beta; zero the consumer operand buffers ----
    float Gv[4][4];  // vector gate: G at (tok 16 it + 4 g + e, f)
    // vector gate, key f: rows 0..3 the centres of the four 16-token windows,
    // rows 4..6 G at tokens 15, 31, 47 and rows 7..9 G at tokens 16, 32, 48
    // (the boundary pivots; kept in LDS, read where used: registers are the
    // scarce resource)
    __shared__ float sWin[VEC ? 10 : 1][DKD];
    float Gnf;
    if (w == 0) sBeta[l] = to_f32(braw);
    if (VEC) {
        float x[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[m][e] = graw[VEC ? 4 * m + e : 0];
        float base = 0.f, mx[4], mn[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
            for (int e = 1; e < 4; ++e) x[m][e] += x[m][e - 1];
            // exclusive prefix over the four row groups of this tile
            const float tot = x[m][3];
            const float p16 = partner16(tot);
            const float pair = tot + p16;
            const float p32 = partner32(pair);
            const float excl = ((g & 1) ? p16 : 0.f) + ((g & 2) ? p32 : 0.f);
            mx[m] = -INFINITY;
            mn[m] = INFINITY;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Gv[m][e] = x[m][e] + excl + base;
                mx[m] = fmaxf(mx[m], Gv[m][e]);
                mn[m] = fminf(mn[m], Gv[m][e]);
            }
            base += pair + p32;
        }
        // G at tokens 63 and 31 (row group 3) and 32 (row group 0) to every row group
        {
            const float pa = partner16(Gv[3][3]);
            const float b1 = (g & 1) ? Gv[3][3] : pa;
            const float pb = partner32(b1);
            Gnf = (g & 2) ? b1 : pb;
        }
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            if (g == 3) sWin[VEC ? 4 + m : 0][f] = Gv[m][3];      // G at token 16 m + 15
            if (g == 0) sWin[VEC ? 7 + m : 0][f] = Gv[m + 1][0];  // G at token 16 m + 16
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float x16 = partner16(mx[h]);
            mx[h] = fmaxf(mx[h], x16);
            const float x32 = partner32(mx[h]);
            mx[h] = fmaxf(mx[h], x32);
            const float n16 = partner16(mn[h]);
            mn[h] = fminf(mn[h], n16);
            const float n32 = partner32(mn[h]);
            mn[h] = fminf(mn[h], n32);
        }
        if (g == 0) {
#pragma unroll
            for (int h = 0; h < 4; ++h) sWin[VEC ? h : 0][f] = 0.5f * (mx[h] + mn[h]);  // window centres
        }
    } else if (w == 0) {
        const float Gl = wave_incl_scan(graw[0]);
        sG[l] = Gl;
        // the consumer loop's per-token factors gam = exp(G) and exp(G_n - G)
        const float Gn = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gl), CH - 1));
        sGam[l] = __expf(Gl);
        sKt[l] = __expf(Gn - Gl);
    }
    auto zero_lG = [&]() {
        const bf16x8 z8 = {};
#pragma unroll
        for (int u = 0; u < (TRG ? 2 : 4); ++u) lG[u * NTHR + tid] = z8;
    };
    if constexpr (!SROW) zero_lG();
    if constexpr (GD2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int id = tid + NTHR * u;
            *(bf16x8*)&sErs[(id >> 4) * EST + (id & 15) * 8] = eraw[u];
        }
    }
    if constexpr (SROW) __builtin_amdgcn_s_waitcnt(0);  // this wave's row and A^T copies have landed
    lds_barrier();
    if constexpr (SROW) {
        // this wave's slices: lane (r, g) takes row 16 m + r, columns 16 w + 4 g .. + 3
        // (16-byte chunk 2 w + g / 2 of the row, its half g & 1)
        auto slice = [&](int mat, int m) -> R4 {
            const int row = 16 * m + r, c = 2 * w + (g >> 1);
            return *(const R4*)(stg + (mat * CH + row) * DKD + (c ^ (row & 15)) * 8 + 4 * (g & 1));
        };
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            vr[m] = rv[m] ? slice(0, m) : R4{};
            orw[m] = rv[m] ? slice(1, m) : R4{};
            kr[m] = rv[m] ? slice(2, m) : R4{};
            qr[m] = rv[m] ? slice(3, m) : R4{};
        }
        lds_barrier();  // every slice is read before phase 1 writes these buffers
        zero_lG();      // (published by the barrier that closes phase 1)
    }
    if (!VEC) Gnf = sG[CH - 1];
    // vector gate, this lane's key: the centre of window m (token tile m);
    // the pivot of row tile m's blocks against earlier windows (G at token
    // 16 m - 1, m >= 1) and against later ones (G at token 16 m + 16, m <= 2)
    auto cen = [&](int m) -> float { return VEC ? sWin[VEC ? m : 0][f] : 0.f; };
    auto piv_lo = [&](int m) -> float { return VEC ? sWin[VEC ? 3 + m : 0][f] : 0.f; };
    auto piv_up = [&](int m) -> float { return VEC ? sWin[VEC ? 7 + m : 0][f] : 0.f; };
    // G at this lane's accumulator position (tok 16 m + 4 g + e, f)
    // G and beta at this lane's accumulator rows (tok 16 m + 4 g + e), read
    // once as 16-byte vectors (the scalar gate's G lives in LDS)
    // (scalar gate only: the vector-gate kernel has no registers to spare
    // and reads beta from LDS where it is used)
    float Gs[VEC ? 1 : 4][4], Bs[VEC ? 1 : 4][4];
    if (!VEC) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float4 b4 = *(const float4*)&sBeta[16 * m + 4 * g];
            const float4 g4 = *(const float4*)&sG[16 * m + 4 * g];
            const float bv[4] = {b4.x, b4.y, b4.z, b4.w}, gv[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Bs[VEC ? 0 : m][e] = bv[e];
                Gs[VEC ? 0 : m][e] = gv[e];
            }
        }
    }
    // G and beta at this lane's accumulator position (tok 16 m + 4 g + e, f)
    auto Gt = [&](int m, int e) -> float { return VEC ? Gv[m][e] : Gs[VEC ? 0 : m][e]; };
    auto Bt = [&](int m, int e) -> float { return VEC ? sBeta[16 * m + 4 * g + e] : Bs[VEC ? 0 : m][e]; };
    // the erase-path weight there: beta, or GDN2's erase gate of (token, key f)
    auto Et = [&](int m, int e) -> float {
        return GD2 ? (float)sErs[(16 * m + 4 * g + e) * EST + f] : Bt(m, e);
    };

    const bf16x8 Ip0k = ident_pi(0, lx);
    const bf16x4 z4 = {};

    if constexpr (SROW) {
#pragma unroll
        for (int j = 0; j < 6; ++j) atf[j] = sAT[j * 64 + l];
    }
    // ---- 1a. P^T = Rb^T A for value tile w ----
    {
        const bf16x8 RbT[2] = {cat8(rbq[0], rbq[1]), cat8(rbq[2], rbq[3])};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // A^T is upper triangular in (i, j): token slab 0 only reaches i < 32
            f32x4 acc = mfma(RbT[1], atf[m], zero4());
            if (m < 2) acc = mfma(RbT[0], atf[4 + m], acc);
            // lane: P[tok 16 m + r][val 16 w + 4 g + e]
            const int i = 16 * m + r;
            const float bt = sBeta[i];
            const f32x4 vx = tof4(vr[m]);
            float dvv[4];
            float pv = 0.f;
            if constexpr (GD2) {
                // dv = wrt o P, dwrt = v o P (entry by entry)
                const f32x4 wx = tof4(wraw[m]);
                float dwv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dvv[e] = wx[e] * acc[e];
                    dwv[e] = vx[e] * acc[e];
                }
                if (i < nv) {
                    store4(dvo + i * ld + 16 * w + 4 * g, dvv);
                    store4((T*)gr.dwrt + tok0 * DVD + i * ld + 16 * w + 4 * g, dwv);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dvv[e] = bt * acc[e];
                    pv += acc[e] * vx[e];
                }
                if (i < nv) store4(dvo + i * ld + 16 * w + 4 * g, dvv);
                pv = sum_rows(pv);
                if (g == 0) sRedP[i][w] = pv;
            }
            if (!WY7) st_half(lP, m * 4 + (w >> 1), w & 1, pack4(acc));
        }
        if (WY7) {
            // Rb fragments (contraction over values) through Rb^T * I, and
            // Z = diag(beta) V fragments, value tile w
            const bf16x8 Ip0 = ident_pi(0, lx), Ip1 = ident_pi(1, lx);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4 cc = mfma(RbT[m >> 1], (m & 1) ? Ip1 : Ip0, zero4());
                st_half(lRb, m * 4 + (w >> 1), w & 1, pack4(cc));
                const f32x4 vx = tof4(vr[m]);
                const float bt = sBeta[16 * m + r];
                bf16x4 z4v;
#pragma unroll
                for (int e = 0; e < 4; ++e) z4v[e] = (bf16)(bt * vx[e]);
                st_half(lZ, m * 4 + (w >> 1), w & 1, z4v);
            }
        }
    }
    // ---- 1b. R and dO fragments (contraction over values) of value tile w ----
    {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // R is stored as ttiles: lane holds R[tok 16 m + r][val 16 w + 4 g + e]
            st_half(lR, m * 4 + (w >> 1), w & 1, rq[m]);
            st_half(lO, m * 4 + (w >> 1), w & 1, tobf4(orw[m]));
        }
    }
    // ---- 1c. h, dh fragments (M = key tile w, K = values); rowsum(h o dh) ----
    if (PF) {
        static_assert(PF_WAIT < 32, "fewer reads than PF_WAIT follow the staging loads");
        asm volatile("s_waitcnt vmcnt(%0)" : : "n"(PF_WAIT) : "memory");  // staged h, dh have landed
#pragma unroll
        for (int vt = 0; vt < 8; ++vt) {
            hq[vt] = area[vt * 64 + l];
            dhq[vt] = area[512 + vt * 64 + l];
        }
    }
    bf16x8 hF[4], dhF[4];
    {
        // ttiles: lane (r, g) holds h[key 16 w + r][val 16 vt + 4 g + e], so
        // value tiles 2 sl and 2 sl + 1 side by side are frag slab sl
        float hdp = 0.f;
#pragma unroll
        for (int vt = 0; vt < 8; ++vt)
#pragma unroll
            for (int e = 0; e < 4; ++e) hdp += (float)hq[vt][e] * (float)dhq[vt][e];
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            hF[sl] = cat8(hq[2 * sl], hq[2 * sl + 1]);
            dhF[sl] = cat8(dhq[2 * sl], dhq[2 * sl + 1]);
        }
        hdp = sum_rows(hdp);  // all 128 values of key 16 w + r
        if (g == 0) sExtra[16 * w + r] = hdp;
    }
    // ---- 1d. K and Q in accumulator order (tok 16 m + 4 g + e, key f) ----
    f32x4 KC[4], QC[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        // the four keys in slots 0..3 are k slots pik(g, 0..3) = 4 g .. 4 g + 3
        // of a 32-wide slab whose upper 16 are zero; the identity in the same
        // pik order maps slot column c < 16 to output column c
        KC[m] = mfma(cat8(tobf4(kr[m]), z4), Ip0k, zero4());
        QC[m] = mfma(cat8(tobf4(qr[m]), z4), Ip0k, zero4());
    }
    // Next chunk's h, dh: requested only now, after the last use of this
    // chunk's reads, so that no wait the compiler places for those reads
    // also waits for the staging loads (they would be younger than the
    // reads in the in-order count). From here on the chunk only stores.
    if (PF && tnext >= 0) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");  // the area has been read
        stage_hdh(it, tnext, w, area);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (WY7) {
        // E = diag(beta)(gam * K) fragments (M = tok, K = key) of key tile w:
        // E^T frags from the K * I accumulators, transposed through E^T * I
        const bf16x8 Ip0 = ident_pi(0, lx), Ip1 = ident_pi(1, lx);
        bf16x8 ETf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            f32x4 ec[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 2 * ks + hh;
                    ec[hh][e] = Bt(m, e) * __expf(Gt(m, e)) * KC[m][e];
                }
            ETf[ks] = pack_pi(ec[0], ec[1]);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // lane: E[tok 16 m + r][key 16 w + 4 g + e]
            const f32x4 cc = mfma(ETf[m >> 1], (m & 1) ? Ip1 : Ip0, zero4());
            st_half(lE, m * 4 + (w >> 1), w & 1, pack4(cc));
        }
    }
    // Consumer B operands (this wave's key tile, K = tokens; token tile m
    // centred at the centre of its window m). Vector gate: the centred factors
    // span exp(+-range/2), and the Gbar terms built from them cancel to far
    // below their size (the diagonal of Hb enters Q'U_q and Y'U_y with
    // opposite signs), so Y', Q', E' are carried as bf16 hi + lo pairs; a
    // single bf16 rounding would dominate dg for strong decays.
    bf16x8 B0[2], B1[2], B2[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        if (VEC) {
            f32x4 y[2], qq[2], ee[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int m = 2 * ks + hh;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = Gt(m, e) - cen(m);
                    const float al = __expf(d), ze = __expf(-d);
                    y[hh][e] = ze * KC[m][e];
                    qq[hh][e] = al * QC[m][e];
                    ee[hh][e] = Et(m, e) * al * KC[m][e];
                }
            }
            B0[ks] = pack_pi(y[0], y[1]);
            B1[ks] = pack_pi(qq[0], qq[1]);
            B2[ks] = pack_pi(ee[0], ee[1]);
            // low parts: x - bf16(x)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    y[hh][e] -= (float)B0[ks][4 * hh + e];
                    qq[hh][e] -= (float)B1[ks][4 * hh + e];
                    ee[hh][e] -= (float)B2[ks][4 * hh + e];
                }
            lo_set(0 * 2 + ks, pack_pi(y[0], y[1]));
            lo_set(1 * 2 + ks, pack_pi(qq[0], qq[1]));
            lo_set(2 * 2 + ks, pack_pi(ee[0], ee[1]));
        } else {
            B0[ks] = pack_pi(KC[2 * ks], KC[2 * ks + 1]);
            B1[ks] = pack_pi(QC[2 * ks], QC[2 * ks + 1]);
            // diag(beta) K, the operand Gam^T multiplies (beta sits on the
            // operand so that D's tiles serve D^T through a transposed read)
            f32x4 bk[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) bk[hh][e] = Bt(2 * ks + hh, e) * KC[2 * ks + hh][e];
            B2[ks] = pack_pi(bk[0], bk[1]);
        }
    }

    lds_barrier();  // lP, lR, lO, sExtra complete

    // ---- 2a'. seven-product producer (ablation): W = Rb h^T (so Wbar = -W),
    //      Abar = Rb Z^T + Wbar E^T, X = A^T Abar; Mbar = -X A^T follows below
    bf16x8 WT[2];  // W^T frags (M = key tile w, K = tok), B operands of Eb_dir
    if (WY7) {
        f32x4 Wc[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 a = zero4(), at = zero4();
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) {
                a = mfma(lRb[(m * 4 + sl) * 64 + l], hF[sl], a);    // W tile (m, w)
                at = mfma(hF[sl], lRb[(m * 4 + sl) * 64 + l], at);  // W^T tile (w, m)
            }
            Wc[m] = a;
            // lane: W^T[key 16 w + 4 g + e][tok 16 m + r] -> W frag (M = tok, K = key)
            st_half(lWb, m * 4 + (w >> 1), w & 1, pack4(at));
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) WT[ks] = pack_pi(Wc[2 * ks], Wc[2 * ks + 1]);
        lds_barrier();  // lWb complete
        // Abar (full 64 x 64), two tiles per wave -> Abar^T frags (M = col, K = row)
        for (int x = w; x < 16; x += NW) {
            const int ta = x >> 2, tb = x & 3;
            f32x4 acc = zero4();
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) acc = mfma(lRb[(ta * 4 + sl) * 64 + l], lZ[(tb * 4 + sl) * 64 + l], acc);
            f32x4 acw = zero4();
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) acw = mfma(lWb[(ta * 4 + sl) * 64 + l], lE[(tb * 4 + sl) * 64 + l], acw);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] -= acw[e];
            // lane: Abar[a = 16 ta + 4 g + e][b = 16 tb + r]
            st_half(lAbT, tb * 2 + (ta >> 1), ta & 1, pack4(acc));
        }
        lds_barrier();  // lAbT complete
        // X^T = Abar^T A (A^T is upper triangular: skip row slab 0 for i >= 32)
        for (int x = w; x < 16; x += NW) {
            const int tc = x >> 2, ti = x & 3;
            f32x4 acc = mfma(lAbT[(tc * 2 + 1) * 64 + l], ld_frag(ATg, ti * 2 + 1), zero4());
            if (ti < 2) acc = mfma(lAbT[(tc * 2 + 0) * 64 + l], ld_frag(ATg, ti * 2 + 0), acc);
            // lane: X[i = 16 ti + r][c = 16 tc + 4 g + e] -> X frag (M = i, K = c)
            st_half(lX, ti * 2 + (tc >> 1), tc & 1, pack4(acc));
        }
        lds_barrier();  // lX complete
    }

    // ---- 2a. D and Hb tiles -> consumer A operands. ReWY:
    //      D = -strict_lower(P R^T). Seven-product: D = strict_lower(Mbar)
    //      with Mbar = -X A^T, formed here as -strict_lower(X A^T). ----
    // One item per 16 x 16 tile of D or Hb, 20 in all (the consumer loop
    // reads D^T and Hb^T from the same tiles, transposed: 40 items before,
    // bwd_local at (1,8192,16) 123.3 -> 114.3 us). The scalar gate's beta,
    // which D^T must not carry, sits on the operand D multiplies instead.
    // The vector-gate seven-product kernel keeps all four kinds of tiles
    // (TRG): with the transposed reads its dk and dg did not repeat from
    // run to run; that kernel spills some 45 registers, and the cause was
    // not found.
    // (scalar gate: the items of a wave unrolled, so that one item's LDS
    // reads overlap the previous item's products; the vector-gate kernel
    // keeps the rolled loop, having no registers to spare)
    auto item2a = [&](int x) {
        // TRG: D (kind 0) and Hb (kind 2); otherwise also D^T (1) and Hb^T (3)
        const int kind = TRG ? 2 * (x / 10) : x / 10, tl = x % 10;
        const int ti = tl >= 6 ? 3 : tl >= 3 ? 2 : tl >= 1 ? 1 : 0;
        const int tj = tl - ti * (ti + 1) / 2;
        f32x4 acc = zero4();
        if (WY7 && kind < 2) {
            // A is lower triangular: its column slab 1 is zero for rows < 32
            const int rj = tj;  // A row tile
            if (kind == 0) {
                // (X A^T)[i][j]: A operand X frag (i), B operand A frag (j)
                acc = mfma(lX[(ti * 2 + 0) * 64 + l], ld_frag(Afg, rj * 2 + 0), acc);
                if (rj >= 2) acc = mfma(lX[(ti * 2 + 1) * 64 + l], ld_frag(Afg, rj * 2 + 1), acc);
            } else {
                // (A X^T)[j][i]
                acc = mfma(ld_frag(Afg, rj * 2 + 0), lX[(ti * 2 + 0) * 64 + l], acc);
                if (rj >= 2) acc = mfma(ld_frag(Afg, rj * 2 + 1), lX[(ti * 2 + 1) * 64 + l], acc);
            }
        } else {
            const bf16x8* Aop = kind == 0 ? lP : kind == 2 ? lO : lR;
            const bf16x8* Bop = kind == 0 ? lR : kind == 1 ? lP : kind == 2 ? lR : lO;
            const int ma = (kind & 1) ? tj : ti, nb = (kind & 1) ? ti : tj;
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) acc = mfma(Aop[(ma * 4 + sl) * 64 + l], Bop[(nb * 4 + sl) * 64 + l], acc);
        }
        // scalar gate: the gate values of this lane's rows and column, as
        // one 16-byte and one 4-byte LDS read
        float4 G4 = {0.f, 0.f, 0.f, 0.f};
        float G1 = 0.f;
        if (!VEC) {
            // kinds 0, 2: lane holds (i = 16 ti + 4 g + e, j = 16 tj + r);
            // kinds 1, 3: (i = 16 ti + r, j = 16 tj + 4 g + e)
            const int i4 = (kind & 1) ? 16 * tj + 4 * g : 16 * ti + 4 * g;
            const int i1 = (kind & 1) ? 16 * ti + r : 16 * tj + r;
            G4 = *(const float4*)&sG[i4];
            G1 = sG[i1];
        }
        const float G4v[4] = {G4.x, G4.y, G4.z, G4.w};
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = (kind & 1) ? 16 * ti + r : 16 * ti + 4 * g + e;
            const int j = (kind & 1) ? 16 * tj + 4 * g + e : 16 * tj + r;
            const bool keep = kind < 2 ? i > j : i >= j;
            float val = keep ? (kind < 2 ? -acc[e] : acc[e]) : 0.f;
            if (!VEC) {
                const float Gi = (kind & 1) ? G1 : G4v[e], Gj = (kind & 1) ? G4v[e] : G1;
                val *= keep ? __expf(Gi - Gj) : 0.f;  // Lam
            }
            o[e] = (bf16)val;
        }
        if constexpr (TRG) {
            if (kind == 0) st_half_tr(lGT, tj * 2 + (ti >> 1), ti & 1, o);  // D:  (M = j, K = i)
            else st_half_tr(lGqT, tj * 2 + (ti >> 1), ti & 1, o);            // Hb: (M = j, K = i)
        } else {
            if (kind == 0) st_half(lGT, tj * 2 + (ti >> 1), ti & 1, o);        // D:    (M = j, K = i)
            else if (kind == 1) st_half(lGm, ti * 2 + (tj >> 1), tj & 1, o);   // D^T:  (M = i, K = j)
            else if (kind == 2) st_half(lGqT, tj * 2 + (ti >> 1), ti & 1, o);  // Hb:   (M = j, K = i)
            else st_half(lGq, ti * 2 + (tj >> 1), tj & 1, o);                  // Hb^T: (M = i, K = j)
        }
    };
    if constexpr (VEC) {
        for (int x = w; x < (TRG ? 20 : 40); x += NW) item2a(x);
    } else if constexpr (PF) {
        // Waves w and w + 4 share a SIMD, and the older one wins its issue
        // slots: waves 4..7 reach every barrier 1.4-2.4k cycles after waves
        // 0..3 (per-wave timestamps). So waves 0..3 take three of the 20
        // items and waves 4..7 two (with the 40 items of four tiles, six and
        // four: bwd_local at (1,8192,16) 135.7 -> 131.5 us; seven and three:
        // 134 us).
        if (w < 4) {
#pragma unroll
            for (int u = 0; u < 3; ++u) item2a(w + 4 * u);
        } else {
#pragma unroll
            for (int u = 0; u < 2; ++u) item2a(12 + (w - 4) + 4 * u);
        }
    } else {
#pragma unroll
        for (int u = 0; u < 3; ++u)
            if (w + NW * u < 20) item2a(w + NW * u);
    }

    lds_barrier();  // consumer A operands complete

    // ---- 2b. Gbar_n extra term: sum_j exp(G_n - G_j) k_j Ktb_j + gam_n rowsum(h o dh) ----
    // The vector gate needs it first (its dg suffix sum starts from it). The
    // scalar gate needs it only at the end of the chunk, so phase 3, which
    // forms the same Kb products, accumulates the sum there instead.
    float colsum = 0.f;
    float extra = 0.f;
    if constexpr (VEC) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f32x4 Kb = zero4();
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) Kb = mfma(lR[(m * 4 + sl) * 64 + l], dhF[sl], Kb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ks = m >> 1, sl = 4 * (m & 1) + e;
                const float kv = ((float)B0[ks][sl] + (float)lo_get(0 * 2 + ks)[sl]) * __expf(Gt(m, e) - cen(m));
                colsum += __expf(Gnf - Gt(m, e)) * kv * Kb[e];
            }
        }
        colsum = sum_rows(colsum);
        extra = colsum + __expf(Gnf) * sExtra[f];
    }

    // ---- 3. per token tile, last to first: producer and state-direct terms,
    //      the four consumer products, chain rules, dq / dk, the per-token
    //      dbeta partials and (vector gate) dg with a running suffix sum ----
    float carry = extra;  // vector gate: suffix sum of Gbar over later tokens
    // bf16 outputs: dq / dk of token tiles 2s and 2s + 1 are turned into rows
    // (4 consecutive keys per lane, one 8-byte store) by one identity product
    // per tile; exact, since each output is a bf16 value times 1.
    constexpr bool ROWSTORE = sizeof(T) == 2;
    f32x4 dqP[2], dkP[2];
    const bf16x8 Ip0 = ident_pi(0, lx), Ip1 = ident_pi(1, lx);
#pragma unroll
    for (int m = 3; m >= 0; --m) {
        // E = P h^T (ReWY) or A^T W with W = Rb h^T (seven-product); both are -Eb_dir
        f32x4 E = zero4(), Qb = zero4(), Kb = zero4();
        if (WY7) {
            E = mfma(ld_frag(ATg, m * 2 + 1), WT[1], E);
            if (m < 2) E = mfma(ld_frag(ATg, m * 2 + 0), WT[0], E);
        }
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            if (!WY7) E = mfma(lP[(m * 4 + sl) * 64 + l], hF[sl], E);
            Qb = mfma(lO[(m * 4 + sl) * 64 + l], hF[sl], Qb);
            Kb = mfma(lR[(m * 4 + sl) * 64 + l], dhF[sl], Kb);
        }
        // lower operands (Gam, Gq: K index <= M index) skip slab 1 for m < 2;
        // upper operands (Gam^T, Gq^T) skip slab 0 for m >= 2
        f32x4 X1 = zero4(), X2 = zero4(), X3 = zero4(), X4 = zero4();
        // vector gate: the blocks against other windows, kept apart since their
        // factors differ: Xa = D Y'x, Xb = Hb Y'x (earlier windows, m >= 1) and
        // Xc = D^T E'x + Hb^T Q'x (later windows, m <= 2); X2 takes both
        // window-centred upper products (they share the factor zeta)
        f32x4 Xa = zero4(), Xb = zero4(), Xc = zero4();
        if constexpr (VEC) {
            // operands against another window from the window-centred ones by a
            // per-key factor at most 1: exp(G[16 m - 1] - c_w) for a window w < m,
            // exp(c_w - G[16 m + 16]) for w > m. (The hi part alone: the
            // cancellation that needs the lo part is in the diagonal blocks.)
            auto rescale4 = [&](const bf16x4& hi, float sc) -> bf16x4 {
                bf16x4 y;
#pragma unroll
                for (int j = 0; j < 4; ++j) y[j] = (bf16)((float)hi[j] * sc);
                return y;
            };
            auto rescale8 = [&](const bf16x8& hi, float s0, float s1) -> bf16x8 {
                return cat8(rescale4(half0(hi), s0), rescale4(half1(hi), s1));
            };
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 0 || m >= 2) {
                    const bf16x8 a1 = TRG ? ld_frag_t64x64(lGT, m, ks) : lGm[(m * 2 + ks) * 64 + l];
                    const bf16x8 a3 = TRG ? ld_frag_t64x64(lGqT, m, ks) : lGq[(m * 2 + ks) * 64 + l];
                    if (ks == (m >> 1) && (m & 1) == 0) {
                        // first half: window m; second half above the diagonal (zero in a1, a3)
                        const bf16x8 lo = lo_get(0 * 2 + ks);
                        X1 = mfma(a1, B0[ks], X1);  // D Y'
                        X3 = mfma(a3, B0[ks], X3);  // Hb Y'
                        X1 = mfma(a1, lo, X1);
                        X3 = mfma(a3, lo, X3);
                    } else if (ks == (m >> 1)) {
                        // first half: window m - 1; second half: window m
                        const bf16x4 lo = half1(lo_get(0 * 2 + ks));
                        X1 = mfma16(half1(a1), half1(B0[ks]), X1);
                        X3 = mfma16(half1(a3), half1(B0[ks]), X3);
                        X1 = mfma16(half1(a1), lo, X1);
                        X3 = mfma16(half1(a3), lo, X3);
                        const bf16x4 yx = rescale4(half0(B0[ks]), __expf(piv_lo(m) - cen(m - 1)));
                        Xa = mfma16(half0(a1), yx, Xa);
                        Xb = mfma16(half0(a3), yx, Xb);
                    } else {
                        // slab 0 for m >= 2: windows 0 and 1, both earlier
                        const float p = piv_lo(m);
                        const bf16x8 yx = rescale8(B0[0], __expf(p - cen(0)), __expf(p - cen(1)));
                        Xa = mfma(a1, yx, Xa);
                        Xb = mfma(a3, yx, Xb);
                    }
                }
                if (ks == 1 || m < 2) {
                    const int ps = TRG ? tr_slot(l) : l;
                    const bf16x8 a2 = lGT[(m * 2 + ks) * 64 + ps], a4 = lGqT[(m * 2 + ks) * 64 + ps];
                    if (ks == (m >> 1) && (m & 1) == 1) {
                        // first half below the diagonal (zero in a2, a4); second half: window m
                        X2 = mfma(a2, B2[ks], X2);  // D^T E'
                        X2 = mfma(a4, B1[ks], X2);  // Hb^T Q'
                        X2 = mfma(a2, lo_get(2 * 2 + ks), X2);
                        X2 = mfma(a4, lo_get(1 * 2 + ks), X2);
                    } else if (ks == (m >> 1)) {
                        // first half: window m; second half: window m + 1
                        X2 = mfma16(half0(a2), half0(B2[ks]), X2);
                        X2 = mfma16(half0(a4), half0(B1[ks]), X2);
                        X2 = mfma16(half0(a2), half0(lo_get(2 * 2 + ks)), X2);
                        X2 = mfma16(half0(a4), half0(lo_get(1 * 2 + ks)), X2);
                        const float sc = __expf(cen(m + 1) - piv_up(m));
                        Xc = mfma16(half1(a2), rescale4(half1(B2[ks]), sc), Xc);
                        Xc = mfma16(half1(a4), rescale4(half1(B1[ks]), sc), Xc);
                    } else {
                        // slab 1 for m < 2: windows 2 and 3, both later
                        const float p = piv_up(m), s2 = __expf(cen(2) - p), s3 = __expf(cen(3) - p);
                        Xc = mfma(a2, rescale8(B2[1], s2, s3), Xc);
                        Xc = mfma(a4, rescale8(B1[1], s2, s3), Xc);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 0 || m >= 2) {
                    const bf16x8 a1 = TRG ? ld_frag_t64x64(lGT, m, ks) : lGm[(m * 2 + ks) * 64 + l];
                    const bf16x8 a3 = TRG ? ld_frag_t64x64(lGqT, m, ks) : lGq[(m * 2 + ks) * 64 + l];
                    X1 = mfma(a1, B0[ks], X1);  // Gam K
                    X3 = mfma(a3, B0[ks], X3);  // Gq K
                }
                if (ks == 1 || m < 2) {
                    const int ps = TRG ? tr_slot(l) : l;
                    const bf16x8 a2 = lGT[(m * 2 + ks) * 64 + ps], a4 = lGqT[(m * 2 + ks) * 64 + ps];
                    X2 = mfma(a2, B2[ks], X2);  // Gam^T diag(beta) K
                    X4 = mfma(a4, B1[ks], X4);  // Gq^T Q
                }
            }
        }
        float Ga[4], br[4];
        float gmv[4] = {0.f, 0.f, 0.f, 0.f}, ktv[4] = {0.f, 0.f, 0.f, 0.f};
        if (!VEC) {
            const float4 gm4 = *(const float4*)&sGam[16 * m + 4 * g], kt4 = *(const float4*)&sKt[16 * m + 4 * g];
            gmv[0] = gm4.x; gmv[1] = gm4.y; gmv[2] = gm4.z; gmv[3] = gm4.w;
            ktv[0] = kt4.x; ktv[1] = kt4.y; ktv[2] = kt4.z; ktv[3] = kt4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * m + 4 * g + e;
            const float G = VEC ? Gt(m, e) : 0.f;
            const float gam = VEC ? __expf(G) : gmv[e], kt = VEC ? __expf(Gnf - G) : ktv[e];
            const float bt = Et(m, e);
            // k and q back from the consumer operands (exact for the scalar
            // gate; hi + lo over the centred factor for the vector gate)
            const int ks = m >> 1, sl = 4 * (m & 1) + e;
            float kv = (float)B0[ks][sl], qv = (float)B1[ks][sl];
            float al = 1.f, ze = 1.f;
            if (VEC) {
                const float d = G - cen(m);  // this row's window
                al = __expf(d);
                ze = __expf(-d);
                kv = (kv + (float)lo_get(0 * 2 + ks)[sl]) * al;
                qv = (qv + (float)lo_get(1 * 2 + ks)[sl]) * ze;
            }
            if (!VEC) colsum += kt * kv * Kb[e];  // the Gbar_n term (phase 2b)
            const float eb = -E[e];  // Eb_dir = -P h^T
            float dq = gam * Qb[e];
            float dk = bt * gam * eb + kt * Kb[e];
            br[e] = gam * kv * eb;
            Ga[e] = gam * qv * Qb[e] + bt * gam * kv * eb - kt * kv * Kb[e];
            if (VEC) {
                // U_q, U_e, U_y with their factors applied
                float uq = al * X3[e], ue = al * X1[e], uy = ze * X2[e];
                if (m >= 1) {
                    const float ax = __expf(G - piv_lo(m));
                    uq += ax * Xb[e];
                    ue += ax * Xa[e];
                }
                if (m <= 2) uy += __expf(piv_up(m) - G) * Xc[e];
                dq += uq;
                dk += bt * ue + uy;
                br[e] += kv * ue;
                Ga[e] += qv * uq + bt * kv * ue - kv * uy;
            } else {
                dq += X3[e];
                dk += bt * X1[e] + X2[e] + X4[e];
                br[e] += kv * X1[e];
                Ga[e] += bt * kv * X1[e] - kv * X2[e] + qv * X3[e] - kv * X4[e];
            }
            if (ROWSTORE) {
                dqP[m & 1][e] = dq;
                dkP[m & 1][e] = dk;
            } else {
                const int off = i * ld + f;
                if (i < nv) {
                    io<T>::st(dqo + off, dq);
                    io<T>::st(dko + off, dk);
                }
            }
        }
        if (ROWSTORE && (m & 1) == 0) {
            // tiles m and m + 1 -> frag (M = key tile w, K = tokens) -> rows
            const bf16x8 aq = pack_pi(dqP[0], dqP[1]), ak = pack_pi(dkP[0], dkP[1]);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                // lane: d*[tok 16 (m + hh) + r][key 16 w + 4 g + e]
                const f32x4 tq = mfma(aq, hh ? Ip1 : Ip0, zero4());
                const f32x4 tk = mfma(ak, hh ? Ip1 : Ip0, zero4());
                const int row = 16 * (m + hh) + r;
                const int off = row * ld + 16 * w + 4 * g;
                float xq[4] = {tq[0], tq[1], tq[2], tq[3]}, xk[4] = {tk[0], tk[1], tk[2], tk[3]};
                if (row < nv) {
                    store4(dqo + off, xq);
                    store4(dko + off, xk);
                }
            }
        }
        if constexpr (GD2) {
            // the erase-gate gradient, entry by entry (what dbeta would sum)
            T* deo = (T*)gr.ders + tok0 * DKD;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * m + 4 * g + e;
                if (i < nv) io<T>::st(deo + i * ld + f, br[e]);
            }
        } else {
            // per-token sums over this wave's features
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float bsum = sum16(br[e]);
                const float gsum = VEC ? 0.f : sum16(Ga[e]);
                if (r == 0) {
                    sRedB[16 * m + 4 * g + e][w] = bsum;
                    if (!VEC) sRedG[16 * m + 4 * g + e][w] = gsum;
                }
            }
        }
        if (VEC) {
            // reverse cumsum down this lane's feature column, tokens 16 m .. 16 m + 15
            float suf[4];
            suf[3] = Ga[3];
#pragma unroll
            for (int e = 2; e >= 0; --e) suf[e] = suf[e + 1] + Ga[e];
            // suffix over the row groups after this one, and the tile total
            const float tot = suf[0];
            const float p16 = partner16(tot);
            const float pair = tot + p16;
            const float p32 = partner32(pair);
            const float excl = ((g & 1) ? 0.f : p16) + ((g & 2) ? 0.f : p32);
            const float ttot = pair + p32;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (16 * m + 4 * g + e < nv) dgo[(16 * m + 4 * g + e) * ld + f] = suf[e] + excl + carry;
            carry += ttot;
        }
        // keep the scheduler from hoisting the next tile's operand reads (the
        // per-chunk kernels, which have no registers to spare; the persistent
        // one, at 240 VGPRs with the hoist, gains 1-2 us at (1,8192,16))
        if (!PF) __builtin_amdgcn_sched_barrier(0);
    }

    // ---- 4. dbeta (wave 1); scalar gate: dg (wave 0), side by side ----
    if (!VEC) {
        colsum = sum_rows(colsum);
        extra = colsum + __expf(Gnf) * sExtra[f];
        const float ex = sum16(extra);
        if (l == 0) sEx[w] = ex;
    }
    lds_barrier();
    if (PF && tnext >= 0) *pend = Tail<T>{dbo, dgo, nv, true};
    else last_phase(dbo, dgo, nv);
}

// Staggered start of the per-chunk launches. Every workgroup begins with about
// 200 KiB of reads and then computes; with one workgroup per CU and all CUs in
// step, each round's reads arrive as one burst. The first workgroup on every
// odd CU (HW_ID.CU_ID, so half the CUs of each shader array) sleeps about
// 6.8 us (2 x 127 x 64 cycles) before it starts, a third of a round. Each CU
// takes its next workgroup when the previous one ends, so the offset carries
// over to the later rounds. ncu_first = the CU count for launches of eight or
// more rounds, else 0 (no delay: a short launch would only lengthen its tail).
__device__ __forceinline__ void staggered_start(int64_t lin, int ncu_first)
{
    if (lin >= ncu_first) return;
    const unsigned cu = __builtin_amdgcn_s_getreg((3 << 11) | (8 << 6) | 4);  // HW_ID bits 8..11
    if (cu & 1u) {
        __builtin_amdgcn_s_sleep(127);
        __builtin_amdgcn_s_sleep(127);
    }
}

template <typename T, bool VEC, bool WY7, bool GD2 = false>
__global__ __launch_bounds__(NTHR) void bwd_local_kernel(Shape s, Inputs in, Inter it, Grads gr, int order,
                                                         int ncu_first)
{
    ChunkRef cr;
    const int64_t lin = blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
    if (!chunk_in_order(s, lin, order, cr))
        return;  // an unused slot of a packed batch
    staggered_start(lin, ncu_first);
    bwd_local_chunk<T, VEC, WY7, false, GD2>(s, in, it, gr, cr, -1, nullptr, nullptr);
}

// Persistent form (scalar gate, three-product producer): workgroup b takes
// items b, b + G, b + 2G, ... of the per-chunk grid (x = chunk or slot
// fastest, then b * H + head; G = gridDim.x) and keeps the next item's h and
// dh streaming into LDS while it works on the current one. With one
// workgroup per CU, a per-chunk launch leaves each CU idle while a new
// workgroup's reads arrive; here those of h and dh (64 KiB of the chunk's
// 169 KiB) arrive during the previous item.
template <typename T>
__global__ __launch_bounds__(NTHR) void bwd_local_pf_kernel(Shape s, Inputs in, Inter it, Grads gr, int order)
{
    __shared__ bf16x4 sStage[NW][STAGE];
    const int64_t NU = slots_used(s), n = NU * (s.B * s.H);  // items in use, dealt evenly
    const int64_t G = gridDim.x;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the item (chunk, head) at or after i that is in use, or i >= n
    auto next_item = [&](int64_t i, ChunkRef& r) -> int64_t {
        ChunkRef x{0, 0, 1};
        while (i < n && !chunk_in_order(s, i, order, NU, x)) i += G;
        if (i < n) r = x;
        return i;
    };
    ChunkRef cur{0, 0, 1};
    int64_t i = next_item(blockIdx.x, cur);
    if (i >= n) return;
    stage_hdh(it, cur.t, w, sStage[w]);
    Tail<T> pend{nullptr, nullptr, 0, false};
    for (;;) {
        ChunkRef nxt{-1, 0, 1};
        const int64_t j = next_item(i + G, nxt);
        bwd_local_chunk<T, false, false, true, false>(s, in, it, gr, cur, j < n ? nxt.t : -1, sStage[w], &pend);
        if (j >= n) break;
        i = j;
        cur = nxt;
    }
}

}  // namespace

hipError_t launch_bwd_local(const Shape& s, const Inputs& in, const Inter& it, const Grads& gr,
                            bool wy7, int order, bool per_chunk, hipStream_t st)
{
    // per-chunk launches: delay half the CUs' first workgroups when the launch
    // runs eight or more rounds of one workgroup per CU
    const int ncu = cu_count();
    const int nf = s.NC * (s.B * s.H) >= 8 * (int64_t)ncu ? ncu : 0;
    if (s.gd2) {
        // GDN2: bf16 inputs, three-product producer only (the host refuses the rest)
        if (s.f32 || !s.vec || wy7) return hipErrorInvalidValue;
        dim3 grid((unsigned)s.NC, (unsigned)(s.B * s.H));
        bwd_local_kernel<bf16, true, false, true><<<grid, NTHR, 0, st>>>(s, in, it, gr, order, nf);
        return hipGetLastError();
    }
    if (!wy7 && !s.vec && !per_chunk) {
        // one workgroup per CU (LDS), each taking every G-th (chunk, head)
        const int64_t n = s.NC * (s.B * s.H);
        if (n <= 0) return hipSuccess;
        const unsigned nb = (unsigned)(n < cu_count() ? n : cu_count());
        if (s.f32) bwd_local_pf_kernel<float><<<nb, NTHR, 0, st>>>(s, in, it, gr, order);
        else bwd_local_pf_kernel<bf16><<<nb, NTHR, 0, st>>>(s, in, it, gr, order);
        return hipGetLastError();
    }
    dim3 grid((unsigned)s.NC, (unsigned)(s.B * s.H));
#define GDR_BWD_LOCAL(W7)                                                                        \
    do {                                                                                         \
        if (s.f32) {                                                                             \
            if (s.vec) bwd_local_kernel<float, true, W7><<<grid, NTHR, 0, st>>>(s, in, it, gr, order, nf); \
            else bwd_local_kernel<float, false, W7><<<grid, NTHR, 0, st>>>(s, in, it, gr, order, nf);      \
        } else {                                                                                 \
            if (s.vec) bwd_local_kernel<bf16, true, W7><<<grid, NTHR, 0, st>>>(s, in, it, gr, order, nf);  \
            else bwd_local_kernel<bf16, false, W7><<<grid, NTHR, 0, st>>>(s, in, it, gr, order, nf);       \
        }                                                                                        \
    } while (0)
    if (wy7) GDR_BWD_LOCAL(true);
    else GDR_BWD_LOCAL(false);
#undef GDR_BWD_LOCAL
    return hipGetLastError();
}

}  // namespace gdr
