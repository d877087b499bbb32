// chunk_prep: per (chunk, head) WY quantities of the chunkwise gated delta rule.
//
// ReWY paper, Sec. 2.3 (the chunk system) and the onedev.kr summary, "How it
// works" (M R = Z - E S with M = I + L, L the strict lower part of E Y^T,
// A = M^{-1}, W = A E, U = A Z). With G the chunk-local inclusive cumsum of
// the log decay, gam = exp(G):
//   E = diag(beta)(gam * K)   Z = diag(beta) V   Y = K / gam
//   L = strict_lower(E Y^T)   Hm = lower_incl((gam * Q) Y^T)
//   Kt = exp(G_n - G) * K     Qg = gam * Q       gn = exp(G_n)
// Scalar gate: E Y^T is beta_i exp(G_i - G_j) (K K^T)_ij, formed from K K^T.
// Vector gate: the centred factors of Sec. 3.3 ("Centered factors"),
// alpha = exp(G - c), zeta = exp(c - G) with c = (max G + min G)/2 per
// feature, give E'Y'^T = E Y^T with every factor bounded by exp(range/2).
// The unit-lower inverse is a 16x16-blocked forward substitution in fp32.
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int LDF = CH + 1;  // fp32 row stride of the 64 x 64 solve buffers

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void prep_kernel(Shape s, Inputs in, Inter it, int write_A)
{
    const int c = blockIdx.x;
    const int bh = blockIdx.y;
    const int64_t b = bh / s.H, h = bh % s.H;
    const int64_t tile = (int64_t)bh * s.NT + c;
    const int64_t tok0 = (b * s.T + (int64_t)c * CH) * s.H + h;  // token of row 0
    const int64_t rs = s.H;                                      // token stride between rows
    const int tid = threadIdx.x;
    const int l = lane_id();
    const int w = wave_id();

    constexpr int GSZ = VEC ? CH * DKD : CH;
    __shared__ float sG[GSZ];
    __shared__ float sCen[DKD];
    __shared__ float sBeta[CH];
    // X region: three 64 x 136 bf16 operand tiles; later the fp32 solve buffers.
    __shared__ __attribute__((aligned(16))) char sX[3 * CH * LD128 * 2];
    __shared__ __attribute__((aligned(16))) bf16 sET[DKD * LD64];  // E^T  [f][i]
    __shared__ __attribute__((aligned(16))) bf16 sZT[DVD * LD64];  // Z^T  [v][i]
    bf16* sX1 = (bf16*)sX;
    bf16* sX2 = sX1 + CH * LD128;
    bf16* sX3 = sX2 + CH * LD128;
    float* sL = (float*)sX;                       // L   fp32 [64][65]
    float* sAi = sL + CH * LDF;                   // A   fp32 [64][65]
    bf16* sAb = (bf16*)(sX + 2 * CH * LD128 * 2); // A   bf16 [64][72]  (in sX3)
    float* sT = (float*)(sAb + CH * LD64);        // 3 x 16 x 17 fp32   (in sX3)

    const T* q = (const T*)in.q;
    const T* k = (const T*)in.k;
    const T* v = (const T*)in.v;
    const T* beta = (const T*)in.beta;

    // ---- 1. gate cumsum (and centre per feature), beta ----
    if (VEC) {
        if (tid < DKD) {
            float acc = 0.f, mx = -INFINITY, mn = INFINITY;
            for (int i = 0; i < CH; ++i) {
                acc += in.g[(tok0 + i * rs) * DKD + tid];
                sG[i * DKD + tid] = acc;
                mx = fmaxf(mx, acc);
                mn = fminf(mn, acc);
            }
            sCen[tid] = 0.5f * (mx + mn);
        }
    } else if (w == 0) {
        float x = in.g[tok0 + l * rs];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            float y = __shfl_up(x, off);
            if (l >= off) x += y;
        }
        sG[l] = x;
    }
    if (tid < CH) sBeta[tid] = io<T>::ld(beta + tok0 + tid * rs);
    __syncthreads();

    // ---- 2. operand tiles ----
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int id = tid + 256 * u;
        const int i = id >> 4;
        const int f0 = (id & 15) * 8;
        const int64_t row = (tok0 + i * rs) * DKD + f0;
        float kx[8], qx[8], vx[8];
        load8(k + row, kx);
        load8(q + row, qx);
        load8(v + row, vx);
        const float bt = sBeta[i];
        float Gi[8], Gn[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            Gi[e] = VEC ? sG[i * DKD + f0 + e] : sG[i];
            Gn[e] = VEC ? sG[(CH - 1) * DKD + f0 + e] : sG[CH - 1];
        }
        float kt[8], qg[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gam = __expf(Gi[e]);
            sET[(f0 + e) * LD64 + i] = (bf16)(bt * gam * kx[e]);
            sZT[(f0 + e) * LD64 + i] = (bf16)(bt * vx[e]);
            kt[e] = __expf(Gn[e] - Gi[e]) * kx[e];
            qg[e] = gam * qx[e];
        }
        store8(it.Kt + (tile * CH + i) * DKD + f0, kt);
        store8(it.Qg + (tile * CH + i) * DKD + f0, qg);
        if (VEC) {
            float ep[8], yp[8], qp[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float cc = sCen[f0 + e];
                const float al = __expf(Gi[e] - cc);
                const float ze = __expf(cc - Gi[e]);
                ep[e] = bt * al * kx[e];
                yp[e] = ze * kx[e];
                qp[e] = al * qx[e];
            }
            *(bf16x8*)(sX1 + i * LD128 + f0) = pack8(ep);
            *(bf16x8*)(sX2 + i * LD128 + f0) = pack8(yp);
            *(bf16x8*)(sX3 + i * LD128 + f0) = pack8(qp);
        } else {
            *(bf16x8*)(sX1 + i * LD128 + f0) = pack8(kx);
            *(bf16x8*)(sX3 + i * LD128 + f0) = pack8(qx);
        }
    }
    if (tid < DKD) it.gn[tile * DKD + tid] = __expf(VEC ? sG[(CH - 1) * DKD + tid] : sG[CH - 1]);
    __syncthreads();

    // ---- 3. L = strict_lower(E Y^T), Hm = lower_incl(Qg Y^T) ----
    f32x4 accL[4], accH[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) { accL[nt] = zero4(); accH[nt] = zero4(); }
    {
        const bf16* Aop = sX1;              // K (scalar) or E' (vector)
        const bf16* Bop = VEC ? sX2 : sX1;  // K (scalar) or Y' (vector)
#pragma unroll
        for (int kk = 0; kk < DKD; kk += 32) {
            bf16x8 aL = frag(Aop, LD128, 16 * w, kk);
            bf16x8 aH = frag(sX3, LD128, 16 * w, kk);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                if (nt <= w) {
                    bf16x8 bb = frag(Bop, LD128, 16 * nt, kk);
                    accL[nt] = mfma(aL, bb, accL[nt]);
                    accH[nt] = mfma(aH, bb, accH[nt]);
                }
            }
        }
    }
    __syncthreads();  // all reads of sX1/sX2/sX3 done before sL/sAi/sAb overwrite them
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const int j = ccol(16 * nt);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = crow(16 * w, r);
            float Lv = 0.f, Hv = 0.f;
            if (nt <= w) {
                float scale = 1.f, bs = 1.f;
                if (!VEC) {
                    scale = __expf(sG[i] - sG[j]);
                    bs = sBeta[i];
                }
                Lv = (i > j) ? accL[nt][r] * scale * bs : 0.f;
                Hv = (i >= j) ? accH[nt][r] * scale : 0.f;
            }
            sL[i * LDF + j] = Lv;
            it.Hm[(tile * CH + i) * CH + j] = (bf16)Hv;
        }
    }
    __syncthreads();

    // ---- 4. A = (I + L)^{-1}: 16x16 diagonal blocks, then block rows ----
    if (l < 16) {
        const int base = 16 * w;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == l) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc -= sL[(base + i) * LDF + base + m] * x[m];
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sAi[(base + i) * LDF + base + l] = x[i];
    }
    __syncthreads();
    {
        const int r = tid >> 4, cc = tid & 15;
        for (int bi = 1; bi < 4; ++bi) {
            // T_bj = sum_{m in [16 bj, 16 bi)} L[16 bi + r][m] A[m][16 bj + cc]
            for (int bj = 0; bj < bi; ++bj) {
                float acc = 0.f;
                for (int m = 16 * bj; m < 16 * bi; ++m)
                    acc += sL[(16 * bi + r) * LDF + m] * sAi[m * LDF + 16 * bj + cc];
                sT[(bj * 16 + r) * 17 + cc] = acc;
            }
            __syncthreads();
            // A[bi][bj] = -A[bi][bi] T_bj
            for (int bj = 0; bj < bi; ++bj) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m)
                    acc += sAi[(16 * bi + r) * LDF + 16 * bi + m] * sT[(bj * 16 + m) * 17 + cc];
                sAi[(16 * bi + r) * LDF + 16 * bj + cc] = -acc;
            }
            __syncthreads();
        }
    }

    // ---- 5. A to bf16 (zero above the diagonal) ----
    for (int e = tid; e < CH * CH; e += 256) {
        const int i = e >> 6, j = e & 63;
        const float a = (j <= i) ? sAi[i * LDF + j] : 0.f;
        sAb[i * LD64 + j] = (bf16)a;
        if (write_A) it.A[(tile * CH + i) * CH + j] = (bf16)a;
    }
    __syncthreads();

    // ---- 6. W = A E, U = A Z ----
    f32x4 aw[4][2], au[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) { aw[mt][nt] = zero4(); au[mt][nt] = zero4(); }
    wave_gemm<4, 2, CH>(sAb, LD64, 0, sET, LD64, 32 * w, aw);
    wave_gemm<4, 2, CH>(sAb, LD64, 0, sZT, LD64, 32 * w, au);
    __syncthreads();  // sET/sZT become staging buffers
    bf16* stW = sET;  // [64][136] fits in 128 x 72
    bf16* stU = sZT;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            put_c(stW, LD128, 16 * mt, 32 * w + 16 * nt, aw[mt][nt]);
            put_c(stU, LD128, 16 * mt, 32 * w + 16 * nt, au[mt][nt]);
        }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int id = tid + 256 * u;
        const int i = id >> 4;
        const int f0 = (id & 15) * 8;
        *(bf16x8*)(it.W + (tile * CH + i) * DKD + f0) = *(const bf16x8*)(stW + i * LD128 + f0);
        *(bf16x8*)(it.U + (tile * CH + i) * DVD + f0) = *(const bf16x8*)(stU + i * LD128 + f0);
    }
}

}  // namespace

hipError_t launch_prep(const Shape& s, const Inputs& in, const Inter& it, bool write_A,
                       hipStream_t st)
{
    dim3 grid((unsigned)s.NT, (unsigned)(s.B * s.H));
    if (s.f32) {
        if (s.vec) prep_kernel<float, true><<<grid, 256, 0, st>>>(s, in, it, write_A);
        else prep_kernel<float, false><<<grid, 256, 0, st>>>(s, in, it, write_A);
    } else {
        if (s.vec) prep_kernel<bf16, true><<<grid, 256, 0, st>>>(s, in, it, write_A);
        else prep_kernel<bf16, false><<<grid, 256, 0, st>>>(s, in, it, write_A);
    }
    return hipGetLastError();
}

}  // namespace gdr
