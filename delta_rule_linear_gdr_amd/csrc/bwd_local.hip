// Chunk-local backward of the chunkwise gated delta rule, one workgroup per
// (chunk, head), after the reverse state scan has produced Rb (the summed
// correction adjoint) and dh (the adjoint of the state at the chunk end).
//
// Producer (ReWY paper, Sec. 3.1, and the onedev.kr summary, "How it works"):
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
//     alpha = exp(G - c), zeta = exp(c - G), c = (max G + min G)/2;
//     U_q = Hb Y', U_e = D Y', U_y = Hb^T Q' + D^T E'  (Y' = zeta K,
//     Q' = alpha Q, E' = beta alpha K);
//     dq += alpha U_q, dk += beta alpha U_e + zeta U_y,
//     dbeta += <U_e, alpha k>, Gbar += Q' U_q + E' U_e - Y' U_y
// Feature-local chain rules for the remaining terms, with gam = exp(G):
//   dq += gam Qgb;  dk += beta gam Eb_dir + exp(G_n - G) Ktb;
//   dbeta += <P, v> + <Eb_dir, gam k>   (undivided, App. B.3)
//   Gbar += gam q Qgb + beta gam k Eb_dir - exp(G_n - G) k Ktb;
//   Gbar_n += sum_j exp(G_n - G_j) k_j Ktb_j + gam_n rowsum(h o dh)
// and dg is the chunk-local reverse cumsum of Gbar (Sec. 3.5), summed over
// features for a scalar gate (App. E.1).
//
// The expanded seven-product producer (Sec. 2.3, "conventional WY
// backward"; onedev.kr: Wb = -Rb S^T, Ab = Rb Z^T + Wb E^T, -A^T Ab A^T) is a
// compile-time variant used only for the ablation; everything after the
// producer is shared.
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int SZ_T128 = CH * LD128 * 2;   // 64 x 136 bf16 = 17408 B
constexpr int SZ_TT = DKD * LD64 * 2;     // 128 x 72 bf16 = 18432 B
constexpr int SZ_T64 = CH * LD64 * 2;     // 64 x 72 bf16  = 9216 B
constexpr int R1_BYTES = 3 * SZ_TT;       // >= 3 * SZ_T128 and >= 64 x 129 fp32
constexpr int R2_BYTES = 4 * SZ_T64;      // >= SZ_T64 + SZ_TT

template <typename T>
__device__ __forceinline__ float ldT(const T* p) { return io<T>::ld(p); }

// Eight waves; wave w owns the 16 feature columns [16w, 16w + 16) of every
// 64 x 128 product (all 64 rows), so the per-element chain rules and the
// gradient accumulators stay in that wave's registers.
constexpr int NWAVE = 8;
constexpr int NTHR = 64 * NWAVE;

template <typename T, bool VEC, bool WY7>
__global__ __launch_bounds__(NTHR) void bwd_local_kernel(Shape s, Inputs in, Inter it, Grads gr)
{
    const int c = blockIdx.x;
    const int bh = blockIdx.y;
    const int64_t b = bh / s.H, h = bh % s.H;
    const int64_t tile = (int64_t)bh * s.NT + c;
    const int64_t tok0 = (b * s.T + (int64_t)c * CH) * s.H + h;
    const int64_t rs = s.H;
    const int tid = threadIdx.x;
    const int l = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int f = 16 * w + (l & 15);  // this lane's feature column in every 64 x 128 product

    constexpr int GSZ = VEC ? CH * DKD : CH;
    __shared__ float sG[GSZ];
    __shared__ float sCen[DKD];
    __shared__ float sBeta[CH];
    __shared__ float sRedB[NWAVE][CH];
    __shared__ float sRedG[NWAVE][CH];
    __shared__ float sExtra[DKD];
    __shared__ __attribute__((aligned(16))) char R1[R1_BYTES];
    __shared__ __attribute__((aligned(16))) char R2[R2_BYTES];
    bf16* Ol = (bf16*)(R1);
    bf16* Rl = (bf16*)(R1 + SZ_T128);
    bf16* Pl = (bf16*)(R1 + 2 * SZ_T128);
    bf16* sAT = (bf16*)(R2);
    bf16* sRbT = (bf16*)(R2 + SZ_T64);
    bf16* C1 = (bf16*)(R2);
    bf16* C2 = (bf16*)(R2 + SZ_T64);
    bf16* C3 = (bf16*)(R2 + 2 * SZ_T64);
    bf16* C4 = (bf16*)(R2 + 3 * SZ_T64);
    bf16* B1 = (bf16*)(R1);
    bf16* B2 = (bf16*)(R1 + SZ_TT);
    bf16* B3 = (bf16*)(R1 + 2 * SZ_TT);

    const T* q = (const T*)in.q;
    const T* k = (const T*)in.k;
    const T* v = (const T*)in.v;
    const T* dO = (const T*)in.dO;
    const T* beta = (const T*)in.beta;
    const bf16* hg = it.h + tile * DKD * DVD;
    const bf16* dhg = it.dh + tile * DKD * DVD;

    // ---- S0: gate cumsum, beta, operand tiles ----
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
    if (tid < CH) sBeta[tid] = ldT(beta + tok0 + tid * rs);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = tid + NTHR * u;
        const int i = id >> 4, f0 = (id & 15) * 8;
        float x[8];
        load8(dO + (tok0 + i * rs) * DVD + f0, x);
        *(bf16x8*)(Ol + i * LD128 + f0) = pack8(x);
        *(bf16x8*)(Rl + i * LD128 + f0) = *(const bf16x8*)(it.R + (tile * CH + i) * DVD + f0);
        const bf16x8 rb = *(const bf16x8*)(it.Rb + (tile * CH + i) * DVD + f0);
#pragma unroll
        for (int e = 0; e < 8; ++e) sRbT[(f0 + e) * LD64 + i] = rb[e];
    }
    {
        const int i = tid >> 3, j0 = (tid & 7) * 8;
        const bf16x8 a = *(const bf16x8*)(it.A + (tile * CH + i) * CH + j0);
#pragma unroll
        for (int e = 0; e < 8; ++e) sAT[(j0 + e) * LD64 + i] = a[e];
    }
    // this lane's q and k entries: rows 16mt + 4(l >> 4) + r, column f
    float qv[4][4], kv[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t off = (tok0 + crow(16 * mt, r) * rs) * DKD + f;
            qv[mt][r] = ldT(q + off);
            kv[mt][r] = ldT(k + off);
        }
    __syncthreads();

    auto Gat = [&](int i) -> float { return VEC ? sG[i * DKD + f] : sG[i]; };
    const float Gnf = VEC ? sG[(CH - 1) * DKD + f] : sG[CH - 1];
    const float cen = VEC ? sCen[f] : 0.f;

    float dq[4][4], dk[4][4], Gacc[4][4], brow[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dq[mt][r] = dk[mt][r] = Gacc[mt][r] = brow[mt][r] = 0.f;
    auto rowi = [&](int mt, int r) { return crow(16 * mt, r); };
    f32x4 X[4][1];
    auto clear = [&]() {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) X[mt][0] = zero4();
    };

    // ---- S1: producer.  P = A^T Rb;  dv = beta P;  dbeta += <P, v> ----
    clear();
    wave_gemm<4, 1, CH>(sAT, LD64, 0, sRbT, LD64, 16 * w, X);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = rowi(mt, r);
            const int64_t off = (tok0 + i * rs) * DVD + f;
            io<T>::st((T*)gr.dv + off, sBeta[i] * X[mt][0][r]);
            brow[mt][r] += X[mt][0][r] * ldT(v + off);
        }
        put_c(Pl, LD128, 16 * mt, 16 * w, X[mt][0]);
    }
    __syncthreads();

    // ---- S2: D = -strict_lower(P R^T) (even waves), Hb = lower_incl(dO R^T)
    //      (odd waves), rows 16 rb .. 16 rb + 15; consumer A operands ----
    {
        const int rb = w >> 1;
        const bool isH = (w & 1) != 0;
        const bf16* Aop = isH ? Ol : Pl;
        f32x4 acc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[nt] = zero4();
#pragma unroll
        for (int kk = 0; kk < DVD; kk += 32) {
            const bf16x8 fa = frag(Aop, LD128, 16 * rb, kk);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
                if (nt <= rb) acc[nt] = mfma(fa, frag(Rl, LD128, 16 * nt, kk), acc[nt]);
        }
        // sAT / sRbT (aliased by C1..C4) were last read in S1, before the barrier.
        bf16* Cn = isH ? C3 : C1;  // [i][j]
        bf16* Ct = isH ? C4 : C2;  // [j][i]
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            const int j = ccol(16 * nt);
            bf16x4 tt;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = crow(16 * rb, r);
                const bool keep = nt <= rb && (isH ? i >= j : i > j);
                float x = keep ? (isH ? acc[nt][r] : -acc[nt][r]) : 0.f;
                float xt = x;
                if (!VEC) {
                    x *= keep ? __expf(sG[i] - sG[j]) : 0.f;   // Gam = D o Lam, Gq = Hb o Lam
                    xt = isH ? x : x * sBeta[i];                // Gam^T diag(beta) as [j][i]
                }
                Cn[i * LD64 + j] = (bf16)x;
                tt[r] = (bf16)xt;
            }
            *(bf16x4*)(Ct + j * LD64 + crow(16 * rb, 0)) = tt;
        }
    }

    // ---- S3: state-direct terms (h, dh read as B operands straight from memory) ----
    {
        // Qgb = dO h^T:  dq += gam X;  Gbar += gam q X
        clear();
        wave_gemm<4, 1, DVD>(Ol, LD128, 0, hg, DVD, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gam = __expf(Gat(rowi(mt, r)));
                dq[mt][r] += gam * X[mt][0][r];
                Gacc[mt][r] += gam * qv[mt][r] * X[mt][0][r];
            }
        // Eb_dir = -P h^T:  dk += beta gam Eb;  dbeta += gam k Eb;  Gbar += beta gam k Eb
        clear();
        wave_gemm<4, 1, DVD>(Pl, LD128, 0, hg, DVD, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rowi(mt, r);
                const float gam = __expf(Gat(i));
                const float eb = -X[mt][0][r];
                const float bt = sBeta[i];
                dk[mt][r] += bt * gam * eb;
                brow[mt][r] += gam * kv[mt][r] * eb;
                Gacc[mt][r] += bt * gam * kv[mt][r] * eb;
            }
        // Ktb = R dh^T:  dk += kt X;  Gbar -= kt k X;  Gbar_n += sum_i kt k X
        float colsum = 0.f;
        clear();
        wave_gemm<4, 1, DVD>(Rl, LD128, 0, dhg, DVD, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float kt = __expf(Gnf - Gat(rowi(mt, r)));
                const float t = kt * X[mt][0][r];
                dk[mt][r] += t;
                Gacc[mt][r] -= kv[mt][r] * t;
                colsum += kv[mt][r] * t;
            }
        colsum += __shfl_xor(colsum, 16);
        colsum += __shfl_xor(colsum, 32);
        // rowsum(h o dh) for this wave's 16 key rows: 4 lanes per row
        float hd = 0.f;
        {
            const int fr = 16 * w + (l >> 2);
            const int v0 = (l & 3) * 32;
#pragma unroll
            for (int e = 0; e < 32; e += 8) {
                const bf16x8 a = *(const bf16x8*)(hg + fr * DVD + v0 + e);
                const bf16x8 bb = *(const bf16x8*)(dhg + fr * DVD + v0 + e);
#pragma unroll
                for (int z = 0; z < 8; ++z) hd += (float)a[z] * (float)bb[z];
            }
            hd += __shfl_xor(hd, 1);
            hd += __shfl_xor(hd, 2);
        }
        if (l < 16) sExtra[f] = colsum;
        __syncthreads();  // sExtra colsums visible; all reads of Ol/Rl/Pl done
        if ((l & 3) == 0) {
            const int fr = 16 * w + (l >> 2);
            const float gn = __expf(VEC ? sG[(CH - 1) * DKD + fr] : sG[CH - 1]);
            sExtra[fr] += gn * hd;
        }
    }

    // ---- S4: consumer B operands (transposed, feature-major) ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = tid + NTHR * u;
        const int j = id >> 4, f0 = (id & 15) * 8;
        float kx[8], qx[8];
        load8(k + (tok0 + j * rs) * DKD + f0, kx);
        load8(q + (tok0 + j * rs) * DKD + f0, qx);
        const float bt = sBeta[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int fe = f0 + e;
            if (VEC) {
                const float cc = sCen[fe];
                const float G = sG[j * DKD + fe];
                const float al = __expf(G - cc), ze = __expf(cc - G);
                B1[fe * LD64 + j] = (bf16)(ze * kx[e]);       // Y'^T
                B2[fe * LD64 + j] = (bf16)(al * qx[e]);       // Q'^T
                B3[fe * LD64 + j] = (bf16)(bt * al * kx[e]);  // E'^T
            } else {
                B1[fe * LD64 + j] = (bf16)kx[e];              // K^T
                B2[fe * LD64 + j] = (bf16)qx[e];              // Q^T
            }
        }
    }
    __syncthreads();

    // ---- S5: consumer products ----
    if (!VEC) {
        // A_K = Gam K
        clear();
        wave_gemm<4, 1, CH>(C1, LD64, 0, B1, LD64, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = X[mt][0][r], bt = sBeta[rowi(mt, r)];
                dk[mt][r] += bt * x;
                brow[mt][r] += kv[mt][r] * x;
                Gacc[mt][r] += bt * kv[mt][r] * x;
            }
        // B_K = Gam^T diag(beta) K,  plus Gq^T Q  (same chain rule)
        clear();
        wave_gemm<4, 1, CH>(C2, LD64, 0, B1, LD64, 16 * w, X);
        wave_gemm<4, 1, CH>(C4, LD64, 0, B2, LD64, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dk[mt][r] += X[mt][0][r];
                Gacc[mt][r] -= kv[mt][r] * X[mt][0][r];
            }
        // Gq K
        clear();
        wave_gemm<4, 1, CH>(C3, LD64, 0, B1, LD64, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dq[mt][r] += X[mt][0][r];
                Gacc[mt][r] += qv[mt][r] * X[mt][0][r];
            }
    } else {
        // U_q = Hb Y'
        clear();
        wave_gemm<4, 1, CH>(C3, LD64, 0, B1, LD64, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float al = __expf(Gat(rowi(mt, r)) - cen);
                dq[mt][r] += al * X[mt][0][r];
                Gacc[mt][r] += al * qv[mt][r] * X[mt][0][r];
            }
        // U_e = D Y'
        clear();
        wave_gemm<4, 1, CH>(C1, LD64, 0, B1, LD64, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = rowi(mt, r);
                const float al = __expf(Gat(i) - cen);
                const float x = X[mt][0][r], bt = sBeta[i];
                dk[mt][r] += bt * al * x;
                brow[mt][r] += al * kv[mt][r] * x;
                Gacc[mt][r] += bt * al * kv[mt][r] * x;
            }
        // U_y = Hb^T Q' + D^T E'
        clear();
        wave_gemm<4, 1, CH>(C4, LD64, 0, B2, LD64, 16 * w, X);
        wave_gemm<4, 1, CH>(C2, LD64, 0, B3, LD64, 16 * w, X);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ze = __expf(cen - Gat(rowi(mt, r)));
                dk[mt][r] += ze * X[mt][0][r];
                Gacc[mt][r] -= ze * kv[mt][r] * X[mt][0][r];
            }
    }

    // ---- S6: outputs ----
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t off = (tok0 + rowi(mt, r) * rs) * DKD + f;
            io<T>::st((T*)gr.dq + off, dq[mt][r]);
            io<T>::st((T*)gr.dk + off, dk[mt][r]);
        }
    // row sums over the wave's features: dbeta (and Gbar for a scalar gate)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float bsum = sum16(brow[mt][r]);
            const float gsum = VEC ? 0.f : sum16(Gacc[mt][r]);
            if ((l & 15) == 0) {
                sRedB[w][rowi(mt, r)] = bsum;
                if (!VEC) sRedG[w][rowi(mt, r)] = gsum;
            }
        }
    __syncthreads();  // all S5 reads of R1 (B1..B3) done; reductions visible
    if (tid < CH) {
        float sb = 0.f;
#pragma unroll
        for (int ww = 0; ww < NWAVE; ++ww) sb += sRedB[ww][tid];
        io<T>::st((T*)gr.dbeta + tok0 + tid * rs, sb);
    }
    if (VEC) {
        float* sGb = (float*)R1;  // [64][129]
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) sGb[rowi(mt, r) * (DKD + 1) + f] = Gacc[mt][r];
        __syncthreads();
        if (tid < DKD) {
            float run = sExtra[tid];
            for (int i = CH - 1; i >= 0; --i) {
                run += sGb[i * (DKD + 1) + tid];
                gr.dg[(tok0 + i * rs) * DKD + tid] = run;
            }
        }
    } else if (w == 0) {
        float ex = sExtra[l] + sExtra[l + 64];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ex += __shfl_xor(ex, off);
        float x = 0.f;
#pragma unroll
        for (int ww = 0; ww < NWAVE; ++ww) x += sRedG[ww][l];
        if (l == CH - 1) x += ex;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(x, off);
            if (l + off < 64) x += y;
        }
        gr.dg[tok0 + l * rs] = x;
    }
}

}  // namespace

hipError_t launch_bwd_local(const Shape& s, const Inputs& in, const Inter& it, const Grads& gr,
                            bool wy7, hipStream_t st)
{
    dim3 grid((unsigned)s.NT, (unsigned)(s.B * s.H));
    if (wy7) return hipErrorNotSupported;
    if (s.f32) {
        if (s.vec) bwd_local_kernel<float, true, false><<<grid, NTHR, 0, st>>>(s, in, it, gr);
        else bwd_local_kernel<float, false, false><<<grid, NTHR, 0, st>>>(s, in, it, gr);
    } else {
        if (s.vec) bwd_local_kernel<bf16, true, false><<<grid, NTHR, 0, st>>>(s, in, it, gr);
        else bwd_local_kernel<bf16, false, false><<<grid, NTHR, 0, st>>>(s, in, it, gr);
    }
    return hipGetLastError();
}

}  // namespace gdr
