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
// The blockIdx -> (head, slice) map keeps the eight slices of a head on one
// XCD so they share its L2. Every slice of a head reads the head's whole
// A1 and A2 (32 KiB per step), so the step time is set by each CU's
// L2-to-CU stream rather than by the arithmetic.
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int NVS = DVD / 16;  // value slices (workgroups) per head

__device__ __forceinline__ void map_block(int nblk, int block, int& bh, int& vs)
{
    int id = block;
    if (nblk % 8 == 0) {
        const int per = nblk / 8;
        id = (id % 8) * per + id / 8;
    }
    bh = id / NVS;
    vs = id % NVS;
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

// One workgroup's walk over the chunks. `block` is its index among the
// B * H * 8 workgroups of this scan.
template <bool BWD, bool OUT, bool STORE, typename T>
__device__ __forceinline__ void scan_body(const Shape& s, const Inputs& in, const Inter& it, T* o,
                                          float* fin, int block)
{
    int bh, vs;
    map_block((int)(s.NS * s.H * NVS), block, bh, vs);
    const SeqView sq = seq_view(s, bh / s.H, bh % s.H);  // bh = sequence * H + head
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
// Loader-fed form of the pair launch. Eight waves per workgroup: waves 0..3
// run the step above; waves 4..7 only move each step's operand tiles from
// global memory into a ring of three LDS slots, two steps ahead, with
// direct-to-LDS loads (global_load_lds_dwordx4: 64 lanes x 16 B = one 1 KiB
// block per instruction, i.e. one frag tile or two ctiles, copied as is).
// The compute waves' instruction streams then carry no global loads, so a
// stall issuing loads behind the shared address unit no longer adds to the
// step's dependent chain (LDS exchange, MFMA, barrier).
//
// Synchronisation uses the two per-step barriers of the step itself:
// slot p % 3 is read by the compute waves in step p; the loaders refill it
// for step p + 3 after the first barrier of step p + 1, and wait for step
// p + 1's blocks before the first barrier of step p + 1.
namespace fed {
constexpr int A1 = 0;           // 16 frag tiles of A1
constexpr int A2 = 16384;       // 16 frag tiles of A2
constexpr int C1 = 32768;       // ctiles 4 vs .. 4 vs + 3 of C1
constexpr int C2 = 34816;       // ctiles 8 vs .. 8 vs + 7 of C2 (reverse)
constexpr int GN = 38912;       // gn (512 B, twice)
constexpr int SLOT = 39936;
constexpr int NSLOT = 3;
constexpr int NB_FWD = 35;      // 1 KiB blocks per step
constexpr int NB_BWD = 39;
constexpr int NL_FWD = (NB_FWD + 3) / 4;  // per loader wave (padded)
constexpr int NL_BWD = (NB_BWD + 3) / 4;
}  // namespace fed

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
template <bool BWD, int J>
__device__ __forceinline__ void fed_issue(const Inter& it, int64_t t, int vs, uint8_t* slot)
{
    constexpr int NB = BWD ? fed::NB_BWD : fed::NB_FWD;
    constexpr int NPAD = (NB + 3) / 4 * 4;
    const int l = lane_id();
    const bf16* A1 = BWD ? it.Kt : it.Wn;
    const bf16* A2 = BWD ? it.WnT : it.KtT;
    const bf16* C1 = BWD ? it.X : it.U;
    // The eight slices of a head read the same A1 / A2 tiles; each starts
    // at a different tile (rotation by 2 vs) so that they do not request
    // the same lines at the same moment.
    const int rot = 2 * vs;
#pragma unroll
    for (int b = J; b < NPAD; b += 4) {
        const void* src;
        int dst;
        if (b < 16) {
            const int bb = (b + rot) & 15;
            src = A1 + t * (CH * DKD) + bb * 512 + l * 8;
            dst = fed::A1 + bb * 1024;
        } else if (b < 32) {
            const int bb = (b - 16 + rot) & 15;
            src = A2 + t * (CH * DKD) + bb * 512 + l * 8;
            dst = fed::A2 + bb * 1024;
        } else if (b < 34) {
            src = C1 + t * (CH * DVD) + vs * 1024 + (b - 32) * 512 + l * 8;
            dst = fed::C1 + (b - 32) * 1024;
        } else if (BWD && b < 38) {
            src = it.Y + t * (DKD * DVD) + vs * 2048 + (b - 34) * 512 + l * 8;
            dst = fed::C2 + (b - 34) * 1024;
        } else {
            src = it.gn + t * DKD + (l & 31) * 4;
            dst = fed::GN;
        }
        lds_dma16(src, slot + dst);
    }
}

template <bool BWD, int J>
__device__ __forceinline__ void fed_loader(const Shape& s, const Inter& it, const SeqView& sq, int vs,
                                           uint8_t* ring)
{
    constexpr int NL = BWD ? fed::NL_BWD : fed::NL_FWD;
    const int NT = (int)sq.nchunk;  // >= 1
    auto issue = [&](int p) {
        const int pc = p < NT ? p : NT - 1;  // past the end: the last chunk again
        const int c = BWD ? NT - 1 - pc : pc;
        fed_issue<BWD, J>(it, seq_tile(s, sq, c), vs, ring + (p % fed::NSLOT) * fed::SLOT);
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

template <bool BWD>
__device__ __forceinline__ void fed_compute(const Shape& s, const Inputs& in, const Inter& it, float* fin,
                                            const SeqView& sq, int bh, int vs, const uint8_t* ring)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id(), r = lane_r(), g = lane_g();
    const int NT = (int)sq.nchunk;  // 0 for an empty sequence: the state passes through
    const int v = 16 * vs + r;

    __shared__ bf16x8 sS[4][64];
    __shared__ bf16x8 sZ[2][64];

    bf16* Sout = BWD ? it.dh : it.h;
    bf16* Zout = BWD ? it.Rb : it.R;
    const float* init = BWD ? in.dht : in.h0;

    f32x4 S[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[m][i] = init ? init[((int64_t)bh * DKD + 32 * w + 16 * m + 4 * g + i) * DVD + v] : 0.f;

    for (int p = 0; p < NT; ++p) {
        const int c = BWD ? NT - 1 - p : p;
        const int64_t t = seq_tile(s, sq, c);
        const uint8_t* slot = ring + (p % fed::NSLOT) * fed::SLOT;
        // state before the update (h_c, or dh_c) as ctiles (key tile 2w + m, value tile vs)
#pragma unroll
        for (int m = 0; m < 2; ++m)
            *(bf16x4*)ctile_ptr(Sout + t * (DKD * DVD), vs * 8 + 2 * w + m) = pack4(S[m]);
        sS[w][l] = pack_pi(S[0], S[1]);
        wait_lgkm0();
        bar();
        bf16x8 sf[4], a1[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            sf[ks] = sS[ks][l];
            a1[ks] = *(const bf16x8*)(slot + fed::A1 + (w * 4 + ks) * 1024 + l * 16);
        }
        // Z = C1 + A1 S   (rows 16w .. 16w + 15)
        f32x4 z = unpack4(*(const bf16x4*)(slot + fed::C1 + (w * 64 + l) * 8));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) z = mfma(a1[ks], sf[ks], z);
        const bf16x4 z4 = pack4(z);
        *(bf16x4*)((bf16*)&sZ[w >> 1][l] + 4 * (w & 1)) = z4;
        wait_lgkm0();
        bar();
        *(bf16x4*)ctile_ptr(Zout + t * (CH * DVD), vs * 4 + w) = z4;
        bf16x8 zf[2], a2[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) zf[ks] = sZ[ks][l];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                a2[m][ks] = *(const bf16x8*)(slot + fed::A2 + ((2 * w + m) * 2 + ks) * 1024 + l * 16);
        // S <- gn S (+ C2) + A2 Z
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const float4 gv = *(const float4*)(slot + fed::GN + (32 * w + 16 * m + 4 * g) * 4);
            f32x4 acc = {gv.x * S[m][0], gv.y * S[m][1], gv.z * S[m][2], gv.w * S[m][3]};
            if (BWD) {
                const f32x4 y = unpack4(*(const bf16x4*)(slot + fed::C2 + ((2 * w + m) * 64 + l) * 8));
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += y[i];
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) acc = mfma(a2[m][ks], zf[ks], acc);
            S[m] = acc;
        }
    }
    if (fin) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fin[((int64_t)bh * DKD + 32 * w + 16 * m + 4 * g + i) * DVD + v] = S[m][i];
    }
}

template <bool BWD>
__device__ __forceinline__ void fed_body(const Shape& s, const Inputs& in, const Inter& it, float* fin,
                                         int block, uint8_t* ring)
{
    int bh, vs;
    map_block((int)(s.NS * s.H * NVS), block, bh, vs);
    const SeqView sq = seq_view(s, bh / s.H, bh % s.H);  // bh = sequence * H + head
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (sq.nchunk == 0 && w >= 4) return;  // an empty sequence: no steps, no barriers
    switch (w) {
    case 4: fed_loader<BWD, 0>(s, it, sq, vs, ring); break;
    case 5: fed_loader<BWD, 1>(s, it, sq, vs, ring); break;
    case 6: fed_loader<BWD, 2>(s, it, sq, vs, ring); break;
    case 7: fed_loader<BWD, 3>(s, it, sq, vs, ring); break;
    default: fed_compute<BWD>(s, in, it, fin, sq, bh, vs, ring); break;
    }
}

// both = 1: the first B*H*8 workgroups walk forward and the next B*H*8
// walk backward side by side (the reverse scan reads only prep's operands,
// not the forward states; each half keeps its XCD mapping, the half size
// being a multiple of 8). both = 0: the reverse scan alone.
__global__ __launch_bounds__(512) void scan_fed_kernel(Shape s, Inputs in, Inter it, float* dh0, int both)
{
    __shared__ __attribute__((aligned(16))) uint8_t ring[fed::NSLOT * fed::SLOT];
    const int nblk = (int)(s.NS * s.H * NVS);
    if (both && (int)blockIdx.x < nblk) fed_body<false>(s, in, it, nullptr, blockIdx.x, ring);
    else fed_body<true>(s, in, it, dh0, both ? blockIdx.x - nblk : blockIdx.x, ring);
}

}  // namespace

hipError_t launch_scan_fwd(const Shape& s, const Inputs& in, const Inter& it, void* o, float* ht,
                           hipStream_t st)
{
    const unsigned nblk = (unsigned)(s.NS * s.H * NVS);
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
    const unsigned nblk = (unsigned)(s.NS * s.H * NVS);
    scan_fed_kernel<<<nblk, 512, 0, st>>>(s, in, it, dh0, 0);
    return hipGetLastError();
}

}  // namespace gdr

namespace gdr {
hipError_t launch_scan_pair(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                            hipStream_t st)
{
    const unsigned nblk = (unsigned)(s.NS * s.H * NVS);
    scan_fed_kernel<<<2 * nblk, 512, 0, st>>>(s, in, it, dh0, 1);
    return hipGetLastError();
}
}  // namespace gdr
