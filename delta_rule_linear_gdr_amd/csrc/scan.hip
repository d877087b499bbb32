// Inter-chunk state scans of the chunkwise gated delta rule.
//
// ReWY paper, Sec. 2.1 and Sec. 3.5 ("The state scan remains serial across
// chunks and parallel across independent value columns"). The state S is
// key-major (128 x 128, fp32 in registers); one workgroup owns BV value
// columns of one head and walks the chunks in order.
//
// Forward, per chunk c (onedev.kr summary, "How it works": R = U - W S):
//   h_c = S;  R_c = U_c - W_c S;  O_c = Qg_c S + Hm_c R_c;
//   S <- diag(gn_c) S + Kt_c^T R_c
// Reverse, per chunk c from last to first, with Sb the adjoint of the state
// at the end of chunk c (paper Sec. 3.1, "State and gate composition": the
// output and next-state adjoints are summed before the local pullback):
//   dh_c = Sb;  Rb_c = Hm_c^T dO_c + Kt_c Sb;
//   Sb <- diag(gn_c) Sb + Qg_c^T dO_c - W_c^T Rb_c
//
// Per-chunk tiles are double-buffered in LDS; the next chunk's tiles are read
// from memory one step ahead. Workgroup -> (head, column slice) mapping keeps
// all slices of a head on one XCD so they share that XCD's L2.
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int BV = 16;         // value columns per workgroup
constexpr int NV = DVD / BV;   // workgroups per head

__device__ __forceinline__ void map_block(int nblk, int& bh, int& vs)
{
    int id = blockIdx.x;
    if (nblk % 8 == 0) {
        const int per = nblk / 8;
        id = (id % 8) * per + id / 8;
    }
    bh = id / NV;
    vs = id % NV;
}

// Read a 64 x 128 bf16 tile: each thread holds 4 chunks of 8 elements.
struct Tile64x128 {
    bf16x8 x[4];
    __device__ void load(const bf16* src)
    {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = threadIdx.x + 256 * u;
            x[u] = *(const bf16x8*)(src + (id >> 4) * 128 + (id & 15) * 8);
        }
    }
    __device__ void store_rows(bf16* dst, int ld) const
    {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = threadIdx.x + 256 * u;
            *(bf16x8*)(dst + (id >> 4) * ld + (id & 15) * 8) = x[u];
        }
    }
    // dst[col][row] (transposed), optionally negated.
    __device__ void store_cols(bf16* dst, int ld, bool neg = false) const
    {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = threadIdx.x + 256 * u;
            const int i = id >> 4, f0 = (id & 15) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[(f0 + e) * ld + i] = neg ? (bf16)(-(float)x[u][e]) : x[u][e];
        }
    }
};

// Read a 64 x 64 bf16 tile: each thread holds 2 chunks of 8 elements.
struct Tile64x64 {
    bf16x8 x[2];
    __device__ void load(const bf16* src)
    {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int id = threadIdx.x + 256 * u;
            x[u] = *(const bf16x8*)(src + (id >> 3) * 64 + (id & 7) * 8);
        }
    }
    __device__ void store_rows(bf16* dst, int ld) const
    {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int id = threadIdx.x + 256 * u;
            *(bf16x8*)(dst + (id >> 3) * ld + (id & 7) * 8) = x[u];
        }
    }
    __device__ void store_cols(bf16* dst, int ld) const
    {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int id = threadIdx.x + 256 * u;
            const int i = id >> 3, j0 = (id & 7) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[(j0 + e) * ld + i] = x[u][e];
        }
    }
};

// ---------------------------------------------------------------- forward

template <typename T>
__global__ __launch_bounds__(256) void scan_fwd_kernel(Shape s, Inputs in, Inter it, T* o, float* ht)
{
    int bh, vs;
    map_block((int)(s.B * s.H * NV), bh, vs);
    const int64_t b = bh / s.H, h = bh % s.H;
    const int v0 = vs * BV;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l = lane_id();
    const bool out = (o != nullptr);

    __shared__ __attribute__((aligned(16))) bf16 sW[2][CH * LD128];
    __shared__ __attribute__((aligned(16))) bf16 sKtT[2][DKD * LD64];
    __shared__ __attribute__((aligned(16))) bf16 sQg[2][CH * LD128];
    __shared__ __attribute__((aligned(16))) bf16 sHm[2][CH * LD64];
    __shared__ __attribute__((aligned(16))) bf16 sSt[BV * LD128];
    __shared__ __attribute__((aligned(16))) bf16 sRt[BV * LD64];

    // state: wave w owns key rows [32w, 32w + 32), two 16-row tiles
    f32x4 S[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int dk = crow(32 * w + 16 * m, r);
            S[m][r] = in.h0 ? in.h0[((int64_t)bh * DKD + dk) * DVD + v0 + ccol(0)] : 0.f;
        }

    Tile64x128 pW, pKt, pQg;
    Tile64x64 pHm;
    auto fetch = [&](int c) {
        const int64_t tile = (int64_t)bh * s.NT + c;
        pW.load(it.W + tile * CH * DKD);
        pKt.load(it.Kt + tile * CH * DKD);
        if (out) {
            pQg.load(it.Qg + tile * CH * DKD);
            pHm.load(it.Hm + tile * CH * CH);
        }
    };
    auto stash = [&](int buf) {
        pW.store_rows(sW[buf], LD128);
        pKt.store_cols(sKtT[buf], LD64);
        if (out) {
            pQg.store_rows(sQg[buf], LD128);
            pHm.store_rows(sHm[buf], LD64);
        }
    };

    fetch(0);
    stash(0);
    if (s.NT > 1) fetch(1);

    for (int c = 0; c < s.NT; ++c) {
        const int cur = c & 1;
        const int64_t tile = (int64_t)bh * s.NT + c;
        // U rows of this wave's R tile, and gn of this wave's key rows
        float u4[4], gnr[2][4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            u4[r] = (float)it.U[(tile * CH + crow(16 * w, r)) * DVD + v0 + ccol(0)];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) gnr[m][r] = it.gn[tile * DKD + crow(32 * w + 16 * m, r)];

        // 1. state to LDS (S^T, bf16) and to memory
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            put_c_t(sSt, LD128, 32 * w + 16 * m, 0, S[m]);
            if (it.h)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    it.h[(tile * DKD + crow(32 * w + 16 * m, r)) * DVD + v0 + ccol(0)] = (bf16)S[m][r];
        }
        __syncthreads();

        // 2. R = U - W S   (rows 16w .. 16w+15)
        f32x4 acc[1][1];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[0][0][r] = -u4[r];
        wave_gemm<1, 1, DKD>(sW[cur], LD128, 16 * w, sSt, LD128, 0, acc);
        f32x4 R;
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = -acc[0][0][r];
        put_c_t(sRt, LD64, 16 * w, 0, R);
        if (it.R)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                it.R[(tile * CH + crow(16 * w, r)) * DVD + v0 + ccol(0)] = (bf16)R[r];
        f32x4 oacc[1][1] = {{zero4()}};
        if (out) wave_gemm<1, 1, DKD>(sQg[cur], LD128, 16 * w, sSt, LD128, 0, oacc);
        __syncthreads();

        // 3. S <- diag(gn) S + Kt^T R ;  O += Hm R
        f32x4 sacc[2][1];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[m][0][r] = S[m][r] * gnr[m][r];
        wave_gemm<2, 1, CH>(sKtT[cur], LD64, 32 * w, sRt, LD64, 0, sacc);
#pragma unroll
        for (int m = 0; m < 2; ++m) S[m] = sacc[m][0];
        if (out) {
            wave_gemm<1, 1, CH>(sHm[cur], LD64, 16 * w, sRt, LD64, 0, oacc);
            const int64_t tok0 = (b * s.T + (int64_t)c * CH) * s.H + h;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                io<T>::st(o + (tok0 + (int64_t)crow(16 * w, r) * s.H) * DVD + v0 + ccol(0), oacc[0][0][r]);
        }

        // 4. next chunk's tiles into the other buffer; fetch the one after
        if (c + 1 < s.NT) {
            stash(cur ^ 1);
            if (c + 2 < s.NT) fetch(c + 2);
        }
    }
    if (ht)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ht[((int64_t)bh * DKD + crow(32 * w + 16 * m, r)) * DVD + v0 + ccol(0)] = S[m][r];
}

// ---------------------------------------------------------------- reverse

template <typename T>
__global__ __launch_bounds__(256) void scan_bwd_kernel(Shape s, Inputs in, Inter it, float* dh0)
{
    int bh, vs;
    map_block((int)(s.B * s.H * NV), bh, vs);
    const int64_t b = bh / s.H, h = bh % s.H;
    const int v0 = vs * BV;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tid = threadIdx.x;

    __shared__ __attribute__((aligned(16))) bf16 sKt[2][CH * LD128];
    __shared__ __attribute__((aligned(16))) bf16 sHT[2][CH * LD64];
    __shared__ __attribute__((aligned(16))) bf16 sQgT[2][DKD * LD64];
    __shared__ __attribute__((aligned(16))) bf16 sWT[2][DKD * LD64];  // holds -W^T
    __shared__ __attribute__((aligned(16))) bf16 sObT[2][BV * LD64];
    __shared__ __attribute__((aligned(16))) bf16 sSbt[BV * LD128];
    __shared__ __attribute__((aligned(16))) bf16 sRbt[BV * LD64];

    f32x4 Sb[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int dk = crow(32 * w + 16 * m, r);
            Sb[m][r] = in.dht ? in.dht[((int64_t)bh * DKD + dk) * DVD + v0 + ccol(0)] : 0.f;
        }

    const T* dO = (const T*)in.dO;
    Tile64x128 pKt, pQg, pW;
    Tile64x64 pHm;
    float pO[8];  // dO slice: threads < 128 hold 8 values of one row
    auto fetch = [&](int c) {
        const int64_t tile = (int64_t)bh * s.NT + c;
        pKt.load(it.Kt + tile * CH * DKD);
        pQg.load(it.Qg + tile * CH * DKD);
        pW.load(it.W + tile * CH * DKD);
        pHm.load(it.Hm + tile * CH * CH);
        if (tid < CH * BV / 8) {
            const int i = tid / (BV / 8), e0 = (tid % (BV / 8)) * 8;
            const int64_t tok = (b * s.T + (int64_t)c * CH + i) * s.H + h;
            load8(dO + tok * DVD + v0 + e0, pO);
        }
    };
    auto stash = [&](int buf) {
        pKt.store_rows(sKt[buf], LD128);
        pQg.store_cols(sQgT[buf], LD64);
        pW.store_cols(sWT[buf], LD64, true);
        pHm.store_cols(sHT[buf], LD64);
        if (tid < CH * BV / 8) {
            const int i = tid / (BV / 8), e0 = (tid % (BV / 8)) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) sObT[buf][(e0 + e) * LD64 + i] = (bf16)pO[e];
        }
    };

    const int NT = (int)s.NT;
    fetch(NT - 1);
    stash((NT - 1) & 1);
    if (NT > 1) fetch(NT - 2);

    for (int c = NT - 1; c >= 0; --c) {
        const int cur = c & 1;
        const int64_t tile = (int64_t)bh * s.NT + c;
        float gnr[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) gnr[m][r] = it.gn[tile * DKD + crow(32 * w + 16 * m, r)];

        // 1. dh_c = Sb
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            put_c_t(sSbt, LD128, 32 * w + 16 * m, 0, Sb[m]);
            if (it.dh)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    it.dh[(tile * DKD + crow(32 * w + 16 * m, r)) * DVD + v0 + ccol(0)] = (bf16)Sb[m][r];
        }
        __syncthreads();

        // 2. Rb = Kt Sb + Hm^T dO   (rows 16w .. 16w+15)
        f32x4 racc[1][1] = {{zero4()}};
        wave_gemm<1, 1, DKD>(sKt[cur], LD128, 16 * w, sSbt, LD128, 0, racc);
        wave_gemm<1, 1, CH>(sHT[cur], LD64, 16 * w, sObT[cur], LD64, 0, racc);
        put_c_t(sRbt, LD64, 16 * w, 0, racc[0][0]);
        if (it.Rb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                it.Rb[(tile * CH + crow(16 * w, r)) * DVD + v0 + ccol(0)] = (bf16)racc[0][0][r];
        __syncthreads();

        // 3. Sb <- diag(gn) Sb + Qg^T dO - W^T Rb
        f32x4 sacc[2][1];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[m][0][r] = Sb[m][r] * gnr[m][r];
        wave_gemm<2, 1, CH>(sQgT[cur], LD64, 32 * w, sObT[cur], LD64, 0, sacc);
        wave_gemm<2, 1, CH>(sWT[cur], LD64, 32 * w, sRbt, LD64, 0, sacc);
#pragma unroll
        for (int m = 0; m < 2; ++m) Sb[m] = sacc[m][0];

        if (c - 1 >= 0) {
            stash(cur ^ 1);
            if (c - 2 >= 0) fetch(c - 2);
        }
    }
    if (dh0)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dh0[((int64_t)bh * DKD + crow(32 * w + 16 * m, r)) * DVD + v0 + ccol(0)] = Sb[m][r];
}

}  // namespace

hipError_t launch_scan_fwd(const Shape& s, const Inputs& in, const Inter& it, void* o, float* ht,
                           hipStream_t st)
{
    const unsigned nblk = (unsigned)(s.B * s.H * NV);
    if (s.f32) scan_fwd_kernel<float><<<nblk, 256, 0, st>>>(s, in, it, (float*)o, ht);
    else scan_fwd_kernel<bf16><<<nblk, 256, 0, st>>>(s, in, it, (bf16*)o, ht);
    return hipGetLastError();
}

hipError_t launch_scan_bwd(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                           hipStream_t st)
{
    const unsigned nblk = (unsigned)(s.B * s.H * NV);
    if (s.f32) scan_bwd_kernel<float><<<nblk, 256, 0, st>>>(s, in, it, dh0);
    else scan_bwd_kernel<bf16><<<nblk, 256, 0, st>>>(s, in, it, dh0);
    return hipGetLastError();
}

}  // namespace gdr
