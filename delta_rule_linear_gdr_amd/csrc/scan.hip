// Inter-chunk state scans of the chunkwise gated delta rule.
//
// ReWY paper (paperpeel.com/paper/2611.01940), Sec. 2.1 and Sec. 3.5: the
// state scan is serial across chunks and parallel across value columns.
// One workgroup owns 16 value columns of one head and walks the chunks; its
// four waves hold the 128 x 16 fp32 state, wave w owning key rows
// [32 w, 32 w + 32) as two accumulator tiles.
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
// frag/ctile order (kernels.h); the only on-chip exchange is the state and
// Z slabs through LDS (one 16-byte write and a few 16-byte reads per lane,
// two barriers). The forward launch (with the output O) prefetches them
// three chunks ahead into registers; the backward launches (the pair, and
// the reverse scan alone) use the loader-fed form further down.
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
// slice vs (NV consecutive value tiles), direction.
struct Chain {
    int64_t n, hd;
    int vs;
    bool bwd;
};

// Workgroups are dealt to the eight XCDs round-robin by index (block b runs
// on XCD b % 8). Chain groups -- the nvs slices of one (sequence, head,
// direction) -- are numbered J = 0, 1, ... and group J goes whole to XCD
// J % 8, so the slices of a group share their A1 / A2 tiles in that XCD's
// L2, and within an XCD the groups start in order of J. In a two-direction
// launch J alternates forward / reverse; the (sequence, head) pairs follow
// s.order (longest sequence first) in packed batches, so the longest walks
// start first. Workgroups past the last group (the grid is rounded up to
// whole rounds of eight groups) have no chain.
__device__ __forceinline__ bool chain_of_block(const Shape& s, int nvs, int ndir, bool bwd1, int block,
                                               Chain& ch)
{
    const int x = block & 7, q = block >> 3;
    const int64_t J = (int64_t)(q / nvs) * 8 + x;
    if (J >= s.NS * s.H * ndir) return false;
    ch.vs = q % nvs;
    ch.bwd = ndir == 2 ? (J & 1) != 0 : bwd1;
    const int64_t j = ndir == 2 ? J >> 1 : J;
    const int64_t k = j / s.H;
    ch.hd = j % s.H;
    ch.n = s.order ? s.order[k] : k;
    return true;
}

unsigned scan_grid(const Shape& s, int nvs, int ndir)
{
    return (unsigned)((s.NS * s.H * ndir + 7) / 8 * 8 * nvs);
}

template <bool BWD, bool OUT>
struct Ops {
    bf16x8 a1[4];     // A1 tiles (mt = w, ks = 0..3)
    bf16x8 a2[2][2];  // A2 tiles (mt = 2w + m, ks = 0..1)
    bf16x4 c1;        // C1 ctile (nt = vs, mt = w)
    bf16x4 c2[2];     // C2 ctiles (nt = vs, mt = 2w + m)      (reverse)
    float4 gn[2];     // gn for keys 32w + 16m + 4g .. +3
    bf16x8 qg[4];     // Qg tiles (mt = w, ks = 0..3)          (output)
    bf16x8 hm[2];     // Hm tiles (mt = w, ks = 0..1)          (output)
};

template <bool BWD, bool OUT>
__device__ __forceinline__ void load_ops(Ops<BWD, OUT>& o, const bf16* A1, const bf16* A2,
                                         const bf16* C1, const bf16* C2, const float* gn,
                                         const bf16* Qg, const bf16* Hm, int64_t t, int w, int vs)
{
    const int g = lane_g();
    const bf16* a1 = A1 + t * (CH * DKD);
    const bf16* a2 = A2 + t * (CH * DKD);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) o.a1[ks] = ld_frag(a1, w * 4 + ks);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o.a2[m][ks] = ld_frag(a2, (2 * w + m) * 2 + ks);
    o.c1 = *(const bf16x4*)ctile_ptr(C1 + t * (CH * DVD), vs * 4 + w);
    if (BWD) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
            o.c2[m] = *(const bf16x4*)ctile_ptr(C2 + t * (DKD * DVD), vs * 8 + 2 * w + m);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) o.gn[m] = *(const float4*)(gn + t * DKD + 32 * w + 16 * m + 4 * g);
    if (OUT) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o.qg[ks] = ld_frag(Qg + t * (CH * DKD), w * 4 + ks);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o.hm[ks] = ld_frag(Hm + t * (CH * CH), w * 2 + ks);
    }
}

// One workgroup's walk over the chunks of one chain.
template <bool BWD, bool OUT, bool STORE, typename T>
__device__ __forceinline__ void scan_body(const Shape& s, const Inputs& in, const Inter& it, T* o,
                                          float* fin, int block)
{
    Chain ch;
    if (!chain_of_block(s, NVS, 1, BWD, block, ch)) return;
    const SeqView sq = seq_view(s, ch.n, ch.hd);
    const int64_t bh = ch.n * s.H + ch.hd;  // state entry
    const int vs = ch.vs;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id(), r = lane_r(), g = lane_g();
    const int NT = (int)sq.nchunk;
    const int v = 16 * vs + r;  // this lane's value column

    __shared__ bf16x8 sS[4][64];  // state slabs: B operands over keys
    __shared__ bf16x8 sZ[2][64];  // Z slabs: B operands over tokens

    const bf16* A1 = BWD ? it.Kt : it.Wn;
    const bf16* A2 = BWD ? it.WnT : it.KtT;
    const bf16* C1 = BWD ? it.X : it.U;
    const bf16* C2 = it.Y;
    bf16* Sout = BWD ? it.dh : it.h;
    bf16* Zout = BWD ? it.Rb : it.R;
    const float* init = BWD ? in.dht : in.h0;

    f32x4 S[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[m][i] = init ? init[((int64_t)bh * DKD + 32 * w + 16 * m + 4 * g + i) * DVD + v] : 0.f;
    auto write_fin = [&]() {
        if (fin) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    fin[((int64_t)bh * DKD + 32 * w + 16 * m + 4 * g + i) * DVD + v] = S[m][i];
        }
    };
    if (NT == 0) {  // an empty sequence of a packed batch: nothing to walk
        write_fin();
        return;
    }

    auto chunk = [&](int p) { return BWD ? NT - 1 - p : p; };
    auto tile = [&](int c) { return seq_tile(s, sq, c); };

    // Stores of a step are issued after the next group of prefetch loads:
    // loads and stores share one in-order completion counter, so a store
    // issued ahead of a prefetch would have to be acknowledged before that
    // prefetch counts as complete.
    bf16x4 pend_s[2], pend_z;
    f32x4 pend_o;
    int64_t pend_t = 0, pend_tok = 0;
    int pend_rows = CH;  // rows of the pending chunk (a ragged last chunk has fewer)
    auto flush = [&]() {
        if (OUT) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * w + 4 * g + i < pend_rows)
                    io<T>::st(o + (pend_tok + (int64_t)i * s.H) * DVD + v, pend_o[i]);
        }
        if (STORE) {
            // state before the update (h_c, or dh_c = adjoint at the chunk
            // end) as ctiles (key tile 2w + m, value tile vs); Z likewise
#pragma unroll
            for (int m = 0; m < 2; ++m)
                *(bf16x4*)ctile_ptr(Sout + pend_t * (DKD * DVD), vs * 8 + 2 * w + m) = pend_s[m];
            *(bf16x4*)ctile_ptr(Zout + pend_t * (CH * DVD), vs * 4 + w) = pend_z;
        }
    };
    auto step = [&](const Ops<BWD, OUT>& op, int c) {
        const int64_t t = tile(c);
        pend_t = t;
        pend_s[0] = pack4(S[0]);
        pend_s[1] = pack4(S[1]);
        sS[w][l] = pack_pi(S[0], S[1]);
        __syncthreads();
        bf16x8 sf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sf[ks] = sS[ks][l];
        // Z = C1 + A1 S   (rows 16w .. 16w + 15)
        f32x4 z = unpack4(op.c1);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) z = mfma(op.a1[ks], sf[ks], z);
        f32x4 oacc = zero4();
        if (OUT) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) oacc = mfma(op.qg[ks], sf[ks], oacc);
        }
        pend_z = pack4(z);
        *(bf16x4*)((bf16*)&sZ[w >> 1][l] + 4 * (w & 1)) = pack4(z);
        __syncthreads();
        bf16x8 zf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) zf[ks] = sZ[ks][l];
        // S <- gn S (+ C2) + A2 Z
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const float gv[4] = {op.gn[m].x, op.gn[m].y, op.gn[m].z, op.gn[m].w};
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gv[i] * S[m][i];
            if (BWD) {
                const f32x4 y = unpack4(op.c2[m]);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += y[i];
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mfma(op.a2[m][ks], zf[ks], acc);
            S[m] = acc;
        }
        if (OUT) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) oacc = mfma(op.hm[ks], zf[ks], oacc);
            pend_tok = seq_tok0(s, sq, c) + (int64_t)(16 * w + 4 * g) * s.H;
            pend_rows = seq_rows(sq, c);
            pend_o = oacc;
        }
    };

    // Three register sets of chunk operands in flight. Every prefetch is
    // issued unconditionally (past the end it re-reads the last chunk), so
    // the number of memory operations per step is fixed and the waits on
    // the vector-memory counter stay exact.
    // The scheduling barriers pin each group of loads where it is written:
    // without them the compiler reorders independent loads across the
    // groups, and the in-order vector-memory counter then makes the first
    // step of every iteration wait for loads issued just before it.
    Ops<BWD, OUT> P0, P1, P2;
    auto load = [&](Ops<BWD, OUT>& op, int p) {
        __builtin_amdgcn_sched_barrier(0);
        load_ops<BWD, OUT>(op, A1, A2, C1, C2, it.gn, it.Qg, it.Hm,
                           tile(chunk(p < NT ? p : NT - 1)), w, vs);
        __builtin_amdgcn_sched_barrier(0);
    };
    load(P0, 0);
    load(P1, 1);
    load(P2, 2);
    int p = 0;
    for (; p + 3 <= NT; p += 3) {
        step(P0, chunk(p));
        load(P0, p + 3);
        flush();
        step(P1, chunk(p + 1));
        load(P1, p + 4);
        flush();
        step(P2, chunk(p + 2));
        load(P2, p + 5);
        flush();
    }
    if (p < NT) {
        step(P0, chunk(p));
        flush();
    }
    if (p + 1 < NT) {
        step(P1, chunk(p + 1));
        flush();
    }
    write_fin();
}

template <bool BWD, bool OUT, bool STORE, typename T>
__global__ __launch_bounds__(256) void scan_kernel(Shape s, Inputs in, Inter it, T* o, float* fin)
{
    scan_body<BWD, OUT, STORE, T>(s, in, it, o, fin, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Loader-fed form of the reverse scan and of the pair launch. Eight waves
// per workgroup: waves 0..3 run the step above; waves 4..7 only move each
// step's operand tiles from global memory into a ring of three LDS slots,
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
// for step p + 3 after the first barrier of step p + 1, and wait for step
// p + 1's blocks before the first barrier of step p + 1.
template <int NV>
struct Fed {
    static constexpr int A1 = 0;                   // 16 frag tiles of A1
    static constexpr int A2 = 16384;               // 16 frag tiles of A2
    static constexpr int C1 = 32768;               // 4 NV ctiles of C1 (value tiles NV vs ..)
    static constexpr int C2 = C1 + NV * 2048;      // 8 NV ctiles of C2 (reverse)
    static constexpr int GN = C2 + NV * 4096;      // gn (512 B, twice)
    static constexpr int SLOT = GN + 1024;
    static constexpr int NSLOT = 3;
    static constexpr int NB_FWD = 32 + 2 * NV + 1;  // 1 KiB blocks per step
    static constexpr int NB_BWD = 32 + 6 * NV + 1;
    static constexpr int NL_FWD = (NB_FWD + 3) / 4;  // per loader wave (padded)
    static constexpr int NL_BWD = (NB_BWD + 3) / 4;
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
// (same bytes to the same place).
template <bool BWD, int J, int NV>
__device__ __forceinline__ void fed_issue(const Inter& it, int64_t t, int vs, uint8_t* slot)
{
    using L = Fed<NV>;
    constexpr int NB = BWD ? L::NB_BWD : L::NB_FWD;
    constexpr int NPAD = (NB + 3) / 4 * 4;
    constexpr int E1 = 32 + 2 * NV, E2 = E1 + 4 * NV;  // ends of the C1 and C2 blocks
    const int l = lane_id();
    const bf16* A1 = BWD ? it.Kt : it.Wn;
    const bf16* A2 = BWD ? it.WnT : it.KtT;
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
            const int bb = (b - 16 + rot) & 15;
            src = A2 + t * (CH * DKD) + bb * 512 + l * 8;
            dst = L::A2 + bb * 1024;
        } else if (b < E1) {
            src = C1 + t * (CH * DVD) + vs * NV * 1024 + (b - 32) * 512 + l * 8;
            dst = L::C1 + (b - 32) * 1024;
        } else if (BWD && b < E2) {
            src = it.Y + t * (DKD * DVD) + vs * NV * 2048 + (b - E1) * 512 + l * 8;
            dst = L::C2 + (b - E1) * 1024;
        } else {
            src = it.gn + t * DKD + (l & 31) * 4;
            dst = L::GN;
        }
        lds_dma16(src, slot + dst);
    }
}

template <bool BWD, int J, int NV>
__device__ __forceinline__ void fed_loader(const Shape& s, const Inter& it, const SeqView& sq, int vs,
                                           uint8_t* ring)
{
    using L = Fed<NV>;
    constexpr int NL = BWD ? L::NL_BWD : L::NL_FWD;
    const int NT = (int)sq.nchunk;  // >= 1
    auto issue = [&](int p) {
        const int pc = p < NT ? p : NT - 1;  // past the end: the last chunk again
        const int c = BWD ? NT - 1 - pc : pc;
        fed_issue<BWD, J, NV>(it, seq_tile(s, sq, c), vs, ring + (p % L::NSLOT) * L::SLOT);
    };
    issue(0);
    issue(1);
    wait_vm<NL>();  // step 0 has landed
    for (int p = 0; p < NT; ++p) {
        bar();  // first barrier of step p: slot (p + 2) % 3 is free
        issue(p + 2);
        bar();  // second barrier of step p
        wait_vm<NL>();  // step p + 1 has landed
    }
    // no LDS write may still be in flight when the workgroup's LDS is released
    wait_vm<0>();
}

// xs: the LDS exchange, NV x 4 state slabs then NV x 2 Z slabs of 64 x 16 B.
template <bool BWD, int NV>
__device__ __forceinline__ void fed_compute(const Shape& s, const Inputs& in, const Inter& it, float* fin,
                                            const SeqView& sq, int64_t bh, int vs, const uint8_t* ring,
                                            bf16x8 (*xs)[64])
{
    using L = Fed<NV>;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id(), r = lane_r(), g = lane_g();
    const int NT = (int)sq.nchunk;  // 0 for an empty sequence: the state passes through
    bf16x8 (*sS)[4][64] = (bf16x8 (*)[4][64])xs;           // [NV][4][64]
    bf16x8 (*sZ)[2][64] = (bf16x8 (*)[2][64])(xs + 4 * NV);  // [NV][2][64]

    bf16* Sout = BWD ? it.dh : it.h;
    bf16* Zout = BWD ? it.Rb : it.R;
    const float* init = BWD ? in.dht : in.h0;

    // state: value tile NV vs + u, key rows 32 w + 16 m + 4 g + i, column 16 (NV vs + u) + r
    f32x4 S[NV][2];
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[u][m][i] = init ? init[(bh * DKD + 32 * w + 16 * m + 4 * g + i) * DVD + 16 * (NV * vs + u) + r]
                                  : 0.f;

    for (int p = 0; p < NT; ++p) {
        const int c = BWD ? NT - 1 - p : p;
        const int64_t t = seq_tile(s, sq, c);
        const uint8_t* slot = ring + (p % L::NSLOT) * L::SLOT;
        // state before the update (h_c, or dh_c) as ctiles (key tile 2w + m, value tile NV vs + u)
#pragma unroll
        for (int u = 0; u < NV; ++u) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
                *(bf16x4*)ctile_ptr(Sout + t * (DKD * DVD), (NV * vs + u) * 8 + 2 * w + m) = pack4(S[u][m]);
            sS[u][w][l] = pack_pi(S[u][0], S[u][1]);
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
            f32x4 z = unpack4(*(const bf16x4*)(slot + L::C1 + ((u * 4 + w) * 64 + l) * 8));
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) z = mfma(a1[ks], sf[u][ks], z);
            z4[u] = pack4(z);
            *(bf16x4*)((bf16*)&sZ[u][w >> 1][l] + 4 * (w & 1)) = z4[u];
        }
        wait_lgkm0();
        bar();
#pragma unroll
        for (int u = 0; u < NV; ++u)
            *(bf16x4*)ctile_ptr(Zout + t * (CH * DVD), (NV * vs + u) * 4 + w) = z4[u];
        bf16x8 zf[NV][2], a2[2][2];
#pragma unroll
        for (int u = 0; u < NV; ++u)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) zf[u][ks] = sZ[u][ks][l];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                a2[m][ks] = *(const bf16x8*)(slot + L::A2 + ((2 * w + m) * 2 + ks) * 1024 + l * 16);
        // S <- gn S (+ C2) + A2 Z
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const float4 gv = *(const float4*)(slot + L::GN + (32 * w + 16 * m + 4 * g) * 4);
#pragma unroll
            for (int u = 0; u < NV; ++u) {
                f32x4 acc = {gv.x * S[u][m][0], gv.y * S[u][m][1], gv.z * S[u][m][2], gv.w * S[u][m][3]};
                if (BWD) {
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

template <bool BWD, int NV>
__device__ __forceinline__ void fed_body(const Shape& s, const Inputs& in, const Inter& it, float* fin,
                                         const Chain& ch, uint8_t* ring, bf16x8 (*xs)[64])
{
    const SeqView sq = seq_view(s, ch.n, ch.hd);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (sq.nchunk == 0 && w >= 4) return;  // an empty sequence: no steps, no barriers
    switch (w) {
    case 4: fed_loader<BWD, 0, NV>(s, it, sq, ch.vs, ring); break;
    case 5: fed_loader<BWD, 1, NV>(s, it, sq, ch.vs, ring); break;
    case 6: fed_loader<BWD, 2, NV>(s, it, sq, ch.vs, ring); break;
    case 7: fed_loader<BWD, 3, NV>(s, it, sq, ch.vs, ring); break;
    default: fed_compute<BWD, NV>(s, in, it, fin, sq, ch.n * s.H + ch.hd, ch.vs, ring, xs); break;
    }
}

// ndir = 2: forward and reverse chains side by side (the reverse scan reads
// only prep's operands, not the forward states); ndir = 1: the reverse scan
// alone. Only the reverse chains write dh0.
template <int NV>
__global__ __launch_bounds__(512) void scan_fed_kernel(Shape s, Inputs in, Inter it, float* dh0, int ndir)
{
    using L = Fed<NV>;
    __shared__ __attribute__((aligned(16))) uint8_t ring[L::NSLOT * L::SLOT];
    __shared__ bf16x8 xs[L::XCH][64];
    Chain ch;
    if (!chain_of_block(s, NVS / NV, ndir, true, blockIdx.x, ch)) return;
    if (ch.bwd) fed_body<true, NV>(s, in, it, dh0, ch, ring, xs);
    else fed_body<false, NV>(s, in, it, nullptr, ch, ring, xs);
}

// Compute units of the current device (cached per device).
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

// One workgroup per CU fits (LDS); NV = 2 when NV = 1 would need more than
// one round of workgroups.
hipError_t launch_fed(const Shape& s, const Inputs& in, const Inter& it, float* dh0, int ndir,
                      hipStream_t st)
{
    if (s.NS * s.H * NVS * ndir > cu_count())
        scan_fed_kernel<2><<<scan_grid(s, NVS / 2, ndir), 512, 0, st>>>(s, in, it, dh0, ndir);
    else
        scan_fed_kernel<1><<<scan_grid(s, NVS, ndir), 512, 0, st>>>(s, in, it, dh0, ndir);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_fwd(const Shape& s, const Inputs& in, const Inter& it, void* o, float* ht,
                           hipStream_t st)
{
    const unsigned nblk = scan_grid(s, NVS, 1);
    const bool store = it.h != nullptr;
    if (o) {
        if (s.f32) {
            if (store) scan_kernel<false, true, true, float><<<nblk, 256, 0, st>>>(s, in, it, (float*)o, ht);
            else scan_kernel<false, true, false, float><<<nblk, 256, 0, st>>>(s, in, it, (float*)o, ht);
        } else {
            if (store) scan_kernel<false, true, true, bf16><<<nblk, 256, 0, st>>>(s, in, it, (bf16*)o, ht);
            else scan_kernel<false, true, false, bf16><<<nblk, 256, 0, st>>>(s, in, it, (bf16*)o, ht);
        }
    } else {
        scan_kernel<false, false, true, bf16><<<nblk, 256, 0, st>>>(s, in, it, nullptr, ht);
    }
    return hipGetLastError();
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
