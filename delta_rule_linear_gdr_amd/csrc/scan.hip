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
// frag/ctile order (kernels.h) and are prefetched three chunks ahead into
// registers; the only on-chip exchange is the state and Z slabs through LDS
// (one 16-byte write and a few 16-byte reads per lane, two barriers).
// The blockIdx -> (head, slice) map keeps the eight slices of a head on one
// XCD so they share its L2.
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
    map_block((int)(s.B * s.H * NVS), block, bh, vs);
    const int64_t b = bh / s.H, hd = bh % s.H;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id(), r = lane_r(), g = lane_g();
    const int NT = (int)s.NT;
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

    auto chunk = [&](int p) { return BWD ? NT - 1 - p : p; };
    auto tile = [&](int c) { return (int64_t)bh * s.NT + c; };

    // Stores of a step are issued after the next group of prefetch loads:
    // loads and stores share one in-order completion counter, so a store
    // issued ahead of a prefetch would have to be acknowledged before that
    // prefetch counts as complete.
    bf16x4 pend_s[2], pend_z;
    f32x4 pend_o;
    int64_t pend_t = 0, pend_tok = 0;
    auto flush = [&]() {
        if (OUT) {
#pragma unroll
            for (int i = 0; i < 4; ++i) io<T>::st(o + (pend_tok + (int64_t)i * s.H) * DVD + v, pend_o[i]);
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
            pend_tok = (b * s.T + (int64_t)c * CH + 16 * w + 4 * g) * s.H + hd;
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
    if (fin) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fin[((int64_t)bh * DKD + 32 * w + 16 * m + 4 * g + i) * DVD + v] = S[m][i];
    }
}

template <bool BWD, bool OUT, bool STORE, typename T>
__global__ __launch_bounds__(256) void scan_kernel(Shape s, Inputs in, Inter it, T* o, float* fin)
{
    scan_body<BWD, OUT, STORE, T>(s, in, it, o, fin, blockIdx.x);
}

// The two scans of the recompute backward in one launch: the reverse scan
// reads only prep's operands (Kt, -W^T, X, Y, gn), not the forward states,
// so the first B*H*8 workgroups walk forward and the next B*H*8 walk
// backward side by side (each half keeps its XCD mapping, the half size
// being a multiple of 8).
__global__ __launch_bounds__(256) void scan_pair_kernel(Shape s, Inputs in, Inter it, float* dh0)
{
    const int nblk = (int)(s.B * s.H * NVS);
    if ((int)blockIdx.x < nblk)
        scan_body<false, false, true, bf16>(s, in, it, nullptr, nullptr, blockIdx.x);
    else
        scan_body<true, false, true, bf16>(s, in, it, nullptr, dh0, blockIdx.x - nblk);
}

}  // namespace

hipError_t launch_scan_fwd(const Shape& s, const Inputs& in, const Inter& it, void* o, float* ht,
                           hipStream_t st)
{
    const unsigned nblk = (unsigned)(s.B * s.H * NVS);
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
    const unsigned nblk = (unsigned)(s.B * s.H * NVS);
    scan_kernel<true, false, true, bf16><<<nblk, 256, 0, st>>>(s, in, it, nullptr, dh0);
    return hipGetLastError();
}

}  // namespace gdr

namespace gdr {
hipError_t launch_scan_pair(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                            hipStream_t st)
{
    const unsigned nblk = (unsigned)(s.B * s.H * NVS);
    scan_pair_kernel<<<2 * nblk, 256, 0, st>>>(s, in, it, dh0);
    return hipGetLastError();
}
}  // namespace gdr
