// chunk_prep: per (chunk, head) quantities of the chunkwise gated delta rule.
//
// ReWY paper (paperpeel.com/paper/2611.01940), Sec. 2.3, and the onedev.kr
// summary, "How it works": the chunk system M R = Z - E S with M = I + L,
// L the strict lower part of E Y^T, A = M^{-1}, W = A E, U = A Z. With G the
// chunk-local inclusive cumsum of the log decay and gam = exp(G):
//   E = diag(beta)(gam * K)   Z = diag(beta) V   Y = K / gam
//   L = strict_lower(E Y^T)   Hm = lower_incl((gam * Q) Y^T)
//   Kt = exp(G_n - G) * K     Qg = gam * Q       gn = exp(G_n)
// Scalar gate: E Y^T = beta_i exp(G_i - G_j) (K K^T)_ij, formed from K K^T.
// Vector gate: the centred factors of Sec. 3.3 ("Centered factors"),
// alpha = exp(G - p), zeta = exp(p - G), give E'Y'^T = E Y^T for any
// per-key pivot p. Each 16 x 16 tile takes its own: a diagonal tile the
// centre (max G + min G)/2 of its 16 rows, a tile below the diagonal G at
// the last row of its column tile (then G_i <= p <= G_j and both factors
// are at most 1 for decays g <= 0). Every factor then stays within
// exp(+-range of 16 tokens / 2), so strong per-token decays stay in fp32
// range where a chunk-wide centre would not.
//
// Work split (four waves): wave w owns keys [32 w, 32 w + 32) and values
// [32 w, 32 w + 32) of every 64 x 128 operand. Transposed operands come from
// an MFMA with the identity (X * I leaves X in accumulator order, which is
// the frag order of X^T), so no operand is transposed through LDS. The
// unit-lower inverse is a 16 x 16-blocked forward substitution in fp32.
// GDN2 (paper Table 1: independent erase and write gates): E = ers o gam o K
// and Z = wrt o V, the erase gate per (token, key) and the write gate per
// (token, value) taking beta's place; both are staged in LDS as fp32.
// Outputs (bit set `what`, formats in kernels.h): the scan operands -W, Kt
// and gn, each once in one orientation (both scan directions read them, the
// transposes through LDS transpose reads), U for the forward scan; the
// output operands Qg, Hm; given dO, X = Hm^T dO and Y = Qg^T dO; Hm^T and
// Qg^T for a later X/Y pass; and A.
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int LP = CH + 4;  // fp32 row stride of the 64 x 64 solve buffers
constexpr int TP = 20;      // fp32 row stride of the 16 x 16 solve temporaries

template <typename T>
__device__ __forceinline__ bf16x8 to_frag(const float (&x)[8])
{
    return pack8(x);
}

// Store 8 consecutive keys (f0 .. f0 + 7, f0 a multiple of 8) of token row
// i as part of a frag (M = 64 tok, K = 128 key) buffer.
__device__ __forceinline__ void st_row8_frag(bf16* base, int i, int f0, const float (&x)[8])
{
    const int ks = f0 >> 5, a = (f0 >> 3) & 3;
    const int tile = (i >> 4) * 4 + ks;
    const int gA = 2 * (a & 1), slot0 = 4 * (a >> 1), r = i & 15;
    bf16x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = (bf16)x[e];
        hi[e] = (bf16)x[4 + e];
    }
    *(bf16x4*)(base + (tile * 64 + 16 * gA + r) * 8 + slot0) = lo;
    *(bf16x4*)(base + (tile * 64 + 16 * (gA + 1) + r) * 8 + slot0) = hi;
}

template <typename T, bool VEC, bool GD2>
__global__ __launch_bounds__(256, 2) void prep_kernel(Shape s, Inputs in, Inter it, int what)
{
    ChunkRef cr;
    // the forward walks chunks 0 .. NC-1; the recompute backward's two walks
    // start at both ends
    const int order = (what & PREP_OUT) ? CO_DESCENDING : CO_MIDDLE_OUT;
    if (!chunk_in_order(s, blockIdx.x + (int64_t)blockIdx.y * gridDim.x, order, cr))
        return;  // an unused slot of a packed batch
    const int64_t t = cr.t;
    const int64_t tok0 = cr.tok0;  // token row of the chunk's row 0
    const int ld = (int)(s.H * DKD);  // row stride (elements); in-chunk offsets < 2^31
    const int nv = cr.nv;  // rows past it are read as zeros
    const int tid = threadIdx.x;
    const int l = lane_id(), r = lane_r(), g = lane_g();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    const bool fwdscan = what & PREP_FWDSCAN, out = what & PREP_OUT, bwdscan = what & PREP_BWDSCAN;
    const bool xy = what & PREP_XY, savexy = what & PREP_SAVEXY, wantA = what & PREP_A;
    const bool walk = fwdscan || bwdscan;  // -W, Kt, gn

    // Vector gate: G per (token, key), rows padded to 132 floats so that the
    // 16 rows a fragment read spans land on distinct LDS banks (a 128-float
    // stride puts them all on the same banks).
    constexpr int GST = DKD + 4;
    constexpr int GSZ = VEC ? CH * GST : CH;
    __shared__ __attribute__((aligned(16))) float sG[GSZ];
    __shared__ float sCen[VEC ? 4 : 1][DKD];  // per 16-row tile: centre of G over its rows
    __shared__ float sBeta[CH];
    // GDN2: the chunk's erase gates (rows 0..63, per key) and write gates
    // (rows 64..127, per value), padded like sG
    __shared__ __attribute__((aligned(16))) float sEW[GD2 ? 2 * CH * GST : 4];
    // L, then A = (I + L)^{-1} in place: block row i reads its L blocks
    // before a barrier and only then writes its A blocks; a diagonal block
    // is read and rewritten by one wave.
    __shared__ __attribute__((aligned(16))) float sL[CH * LP];
    float* const sA = sL;
    __shared__ __attribute__((aligned(16))) float sT[3 * 16 * TP];
    __shared__ bf16x8 sHmT[8 * 64];   // Hm^T frag (M = 64 tok j, K = 64 tok i)
    __shared__ bf16x8 sQgT[16 * 64];  // Qg^T frag (M = 128 key, K = 64 tok)

    const T* q = (const T*)in.q + tok0 * DKD;
    const T* k = (const T*)in.k + tok0 * DKD;
    const T* v = (const T*)in.v + tok0 * DVD;
    const T* dO = (const T*)in.dO + tok0 * DVD;
    const T* beta = (const T*)in.beta;

    // bf16 scalar-gate path: the chunk's K and Q rows are copied once into
    // LDS (64 rows x 256 B each; 16-byte chunk j of row i stored at chunk
    // j ^ (i & 15), so fragment reads over 16 rows and row reads over 16
    // chunks are both free of bank conflicts) and every later K / Q read
    // comes from there. Direct-to-LDS loads: instruction b of wave w covers
    // rows 4 (b & 15) .. + 3 of K (b < 16) or Q, lane L landing at row
    // 4 (b & 15) + L / 16, stored chunk L % 16.
    constexpr bool STAGE = sizeof(T) == 2 && !VEC;
    __shared__ __attribute__((aligned(16))) bf16 sKQ[STAGE ? 2 * CH * DKD : 8];
    if (STAGE) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int b = w * 8 + i, mat = b >> 4, row = 4 * (b & 15) + (l >> 4);
            const int chunk = (l & 15) ^ (row & 15);
            const T* src = (mat ? q : k) + row * ld + chunk * 8;
            bf16* dst = sKQ + mat * CH * DKD + 4 * (b & 15) * DKD;
            if (row < nv) lds_dma16(src, dst);
            else *(bf16x8*)(dst + l * 8) = bf16x8{};
        }
    }

    // ---- 1. gate cumsum (and per-key centre), beta ----
    // (beta and a scalar gate are read by every wave, so that no branch has
    // to wait for them)
    // Rows past nv: the read is made from a clamped row (always in range, so
    // it stays an unconditional read in the batch) and its value replaced by
    // zero with a select.
    // gate check: this lane's log decays and (vector gate) window ranges
    bool gpos = false, gnonfin = false, grange = false;
    const int lc = l < nv ? l : nv - 1;
    const T bload = GD2 ? (T)0.f : beta[tok0 + lc * s.H];
    const float gload = VEC ? 0.f : in.g[tok0 + lc * s.H];
    const T braw = l < nv ? bload : (T)0.f;
    const float graw = l < nv ? gload : 0.f;
    if (VEC) {
        // wave w: keys 32 w .. 32 w + 31 as two 16-key passes; lane (r, g)
        // holds tokens 16 m + 4 g + e of key f (all 32 reads issued first)
        float x[2][4][4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * m + 4 * g + e, ic = i < nv ? i : nv - 1;
                    x[u][m][e] = in.g[(tok0 + (int64_t)ic * s.H) * DKD + 32 * w + 16 * u + r];
                }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x[u][m][e] = 16 * m + 4 * g + e < nv ? x[u][m][e] : 0.f;
                    gpos |= x[u][m][e] > 0.f;
                    gnonfin |= !__builtin_isfinite(x[u][m][e]);
                }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int f = 32 * w + 16 * u + r;
            float base = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int e = 1; e < 4; ++e) x[u][m][e] += x[u][m][e - 1];
                // exclusive prefix over the four row groups of this tile
                const float tot = x[u][m][3];
                const float p16 = partner16(tot);
                const float pair = tot + p16;
                const float p32 = partner32(pair);
                const float excl = ((g & 1) ? p16 : 0.f) + ((g & 2) ? p32 : 0.f);
                float mx = -INFINITY, mn = INFINITY;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float G = x[u][m][e] + excl + base;
                    sG[(16 * m + 4 * g + e) * GST + f] = G;
                    mx = fmaxf(mx, G);
                    mn = fminf(mn, G);
                }
                base += pair + p32;
                // centre of this 16-row tile
                const float mx16 = partner16(mx);
                mx = fmaxf(mx, mx16);
                const float mx32 = partner32(mx);
                mx = fmaxf(mx, mx32);
                const float mn16 = partner16(mn);
                mn = fminf(mn, mn16);
                const float mn32 = partner32(mn);
                mn = fminf(mn, mn32);
                if (g == 0) sCen[VEC ? m : 0][f] = 0.5f * (mx + mn);
                grange |= mx - mn > GATE_RANGE_MAX;
            }
        }
    } else if (w == 0) {
        sG[l] = wave_incl_scan(graw);
        gpos = graw > 0.f;
        gnonfin = !__builtin_isfinite(graw);
    }
    if (it.flags) {
        // every prep run rewrites all four words of its (chunk, head)
        const uint32_t bits = (__ballot(gpos) ? (uint32_t)GATE_POSITIVE : 0u) |
                              (__ballot(grange) ? (uint32_t)GATE_RANGE : 0u) |
                              (__ballot(gnonfin) ? (uint32_t)GATE_NONFINITE : 0u);
        if (l == 0) it.flags[t * 4 + w] = bits;
    }
    if (w == 0) sBeta[l] = to_f32(braw);
    if constexpr (GD2) {
        // 64 rows x 128 of each gate as groups of four; rows past nv are zero
        const T* ers = (const T*)in.ers + tok0 * DKD;
        const T* wrt = (const T*)in.wrt + tok0 * DVD;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int id = tid + 256 * u, i = id >> 5, c = (id & 31) * 4;
            const int ic = i < nv ? i : nv - 1;
            const f32x4 e4 = tof4(ld4raw(ers + ic * ld + c)), w4 = tof4(ld4raw(wrt + ic * ld + c));
            *(f32x4*)&sEW[i * GST + c] = i < nv ? e4 : zero4();
            *(f32x4*)&sEW[(CH + i) * GST + c] = i < nv ? w4 : zero4();
        }
    }
    if (STAGE) __builtin_amdgcn_s_waitcnt(0);  // the K / Q copies have landed
    lds_barrier();

    auto Gat = [&](int i, int f) -> float { return VEC ? sG[i * GST + f] : sG[i]; };
    if (walk && tid < DKD) it.gn[t * DKD + tid] = __expf(Gat(CH - 1, tid));

    // plain fragment of row block i0 .. i0+15, keys 32 ks + 8 g .. + 7: the
    // unconverted read, then the bf16 operand with an optional per-(row, key)
    // scale (vector gate)
    typedef decltype(ld8raw(k)) R8;
    auto raw_rows = [&](const T* base, int i0, int ks) -> R8 {
        const int i = i0 + r;
        const R8 x = ld8raw(base + (i < nv ? i : nv - 1) * ld + 32 * ks + 8 * g);
        return i < nv ? x : R8{};
    };
    // 16-byte chunk j of row i of staged K (mat 0) or Q (mat 1)
    auto kq_chunk = [&](int mat, int i, int j) -> bf16x8 {
        return *(const bf16x8*)(sKQ + mat * CH * DKD + i * DKD + ((j ^ (i & 15)) * 8));
    };
    auto raw_k = [&](int i0, int ks) -> R8 {
        if constexpr (STAGE) return kq_chunk(0, i0 + r, 4 * ks + g);
        else return raw_rows(k, i0, ks);
    };
    auto raw_q = [&](int i0, int ks) -> R8 {
        if constexpr (STAGE) return kq_chunk(1, i0 + r, 4 * ks + g);
        else return raw_rows(q, i0, ks);
    };
    // pv: the tile pair's per-key pivot (vector gate)
    auto cook = [&](const R8& raw, int i0, int ks, int kind, const float* pv) -> bf16x8 {
        if (!VEC || kind == 0) return tobf8(raw);
        float x[8];
        to_f8(raw, x);
        const int i = i0 + r, f0 = 32 * ks + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float d = sG[i * GST + f0 + e] - pv[f0 + e];
            // 1: alpha = exp(G - p) (queries);  2: beta alpha (erase keys);
            // 3: zeta = exp(p - G) (write keys)
            const float wgt = GD2 ? sEW[i * GST + f0 + e] : sBeta[i];  // erase weight
            x[e] *= (kind == 3) ? __expf(-d) : __expf(d) * (kind == 2 ? wgt : 1.f);
        }
        return pack8(x);
    };

    // ---- 2. L = strict_lower(E Y^T) and Hm = lower_incl(Qg Y^T), 16 x 16 tiles ----
    {
        const bool needH = xy || savexy, needHt = out;
        // lower 16 x 16 tiles (ti, tj <= ti) in row order; wave w takes tiles
        // w, w + 4, w + 8 and reads the next tile's fragments before it
        // computes the current one
        auto tile_ij = [](int x, int& ti, int& tj) {
            ti = x >= 6 ? 3 : x >= 3 ? 2 : x >= 1 ? 1 : 0;
            tj = x - ti * (ti + 1) / 2;
        };
        R8 buf[2][3][4];  // [parity][K rows ti, K rows tj, Q rows ti][ks]
        auto read_tile = [&](int x, R8 (&b)[3][4]) {
            int ti, tj;
            tile_ij(x, ti, tj);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                b[0][ks] = raw_k(16 * ti, ks);
                b[1][ks] = raw_k(16 * tj, ks);
                b[2][ks] = raw_q(16 * ti, ks);
            }
        };
        read_tile(w, buf[0]);
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int x = w + 4 * u;
            if (x >= 10) break;
            // (unconditional, the last tile again past the end, so that the
            // waits on the in-order memory counter stay exact)
            read_tile(x + 4 < 10 ? x + 4 : 9, buf[(u + 1) & 1]);
            int ti, tj;
            tile_ij(x, ti, tj);
            const R8(&b)[3][4] = buf[u & 1];
            // vector gate: the centre of a diagonal tile, else G at the last
            // row of the column tile
            const float* pv = ti == tj ? sCen[VEC ? ti : 0] : &sG[VEC ? (16 * tj + 15) * GST : 0];
            f32x4 aL = zero4(), aH = zero4(), aHt = zero4();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 ki = cook(b[0][ks], 16 * ti, ks, 2, pv);  // E' rows (scalar: K)
                const bf16x8 kj = cook(b[1][ks], 16 * tj, ks, 3, pv);  // Y' rows (scalar: K)
                aL = mfma(ki, kj, aL);
                if (needH || needHt) {
                    const bf16x8 qi = cook(b[2][ks], 16 * ti, ks, 1, pv);  // Q' rows (scalar: Q)
                    if (needH) aH = mfma(qi, kj, aH);
                    if (needHt) aHt = mfma(kj, qi, aHt);
                }
            }
            // aL, aH: lane holds (i = 16 ti + 4 g + e, j = 16 tj + r)
            // aHt:    lane holds (j = 16 tj + 4 g + e, i = 16 ti + r)
            bf16x4 hv, htv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * ti + 4 * g + e, j = 16 * tj + r;
                float lam = 1.f, bs = 1.f;
                if (!VEC) {
                    lam = __expf(sG[i] - sG[j]);
                    bs = sBeta[i];
                }
                sL[i * LP + j] = (i > j) ? aL[e] * lam * bs : 0.f;
                hv[e] = (bf16)((i >= j) ? aH[e] * lam : 0.f);
                const int i2 = 16 * ti + r, j2 = 16 * tj + 4 * g + e;
                const float lam2 = VEC ? 1.f : __expf(sG[i2] - sG[j2]);
                htv[e] = (bf16)((i2 >= j2) ? aHt[e] * lam2 : 0.f);
            }
            // Hm^T frag (M = j, K = i): tile (tj, ti >> 1), half ti & 1
            const int hoff = (((tj * 2 + (ti >> 1)) * 64 + l) * 8) + 4 * (ti & 1);
            if (xy) *(bf16x4*)((bf16*)sHmT + hoff) = hv;
            if (savexy) *(bf16x4*)(it.HmT + t * (CH * CH) + hoff) = hv;
            // Hm frag (M = i, K = j): tile (ti, tj >> 1), half tj & 1
            if (out)
                *(bf16x4*)(it.Hm + t * (CH * CH) + (((ti * 2 + (tj >> 1)) * 64 + l) * 8) + 4 * (tj & 1)) =
                    htv;
        }
        // the zero halves / tiles of the two triangular frag buffers
        if (w == 0) {
            const bf16x4 z4 = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            const bf16x8 z8 = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f,
                               (bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
            // Hm^T: (tj=1, ti=0) and (tj=3, ti=2) halves; tiles (tj=2,3; ks=0)
            if (xy || savexy) {
                bf16* dst = xy ? (bf16*)sHmT : it.HmT + t * (CH * CH);
                if (xy && savexy) {
                    // both: write the global copy too
                    bf16* g2 = it.HmT + t * (CH * CH);
                    *(bf16x4*)(g2 + ((1 * 2 + 0) * 64 + l) * 8) = z4;
                    *(bf16x4*)(g2 + ((3 * 2 + 1) * 64 + l) * 8) = z4;
                    *(bf16x8*)(g2 + ((2 * 2 + 0) * 64 + l) * 8) = z8;
                    *(bf16x8*)(g2 + ((3 * 2 + 0) * 64 + l) * 8) = z8;
                }
                *(bf16x4*)(dst + ((1 * 2 + 0) * 64 + l) * 8) = z4;
                *(bf16x4*)(dst + ((3 * 2 + 1) * 64 + l) * 8) = z4;
                *(bf16x8*)(dst + ((2 * 2 + 0) * 64 + l) * 8) = z8;
                *(bf16x8*)(dst + ((3 * 2 + 0) * 64 + l) * 8) = z8;
            }
            // Hm: (ti=0, tj=1) and (ti=2, tj=3) halves; tiles (ti=0,1; ks=1)
            if (out) {
                bf16* dst = it.Hm + t * (CH * CH);
                *(bf16x4*)(dst + ((0 * 2 + 0) * 64 + l) * 8 + 4) = z4;
                *(bf16x4*)(dst + ((2 * 2 + 1) * 64 + l) * 8 + 4) = z4;
                *(bf16x8*)(dst + ((0 * 2 + 1) * 64 + l) * 8) = z8;
                *(bf16x8*)(dst + ((1 * 2 + 1) * 64 + l) * 8) = z8;
            }
        }
    }

    // ---- reads of phases 4 and 4b, issued now so that they land during the
    //      solve: K, V, dO, Q fragments of slab w, and four K and Q row pieces
    //      per thread (dO is read only when X, Y are made; otherwise Q again) ----
    R8 rk[4], rv[4], ro[4], rq[4], rkr[4], rqr[4];
    {
        const T* dOs = xy ? dO : q;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            rk[mt] = raw_k(16 * mt, w);
            rv[mt] = raw_rows(v, 16 * mt, w);
            ro[mt] = raw_rows(dOs, 16 * mt, w);
            rq[mt] = raw_q(16 * mt, w);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = tid + 256 * u;
            const int i = id >> 4, f0 = (id & 15) * 8;
            if constexpr (STAGE) {
                rkr[u] = kq_chunk(0, i, id & 15);
                rqr[u] = kq_chunk(1, i, id & 15);
            } else {
                const int ic = i < nv ? i : nv - 1;
                const R8 xk = ld8raw(k + ic * ld + f0), xq = ld8raw(q + ic * ld + f0);
                rkr[u] = i < nv ? xk : R8{};
                rqr[u] = i < nv ? xq : R8{};
            }
        }
    }

    lds_barrier();  // sL complete

    // ---- 3. A = (I + L)^{-1}: diagonal 16 x 16 blocks, then block rows ----
    {
        // zero the upper blocks of sA
        for (int e = tid; e < 6 * 256; e += 256) {
            // upper blocks (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)
            const int bk = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            const int bi = bk < 3 ? 0 : bk < 5 ? 1 : 2;
            const int bj = bi == 0 ? bk + 1 : bi == 1 ? bk - 1 : 3;
            sA[(16 * bi + rr) * LP + 16 * bj + cc] = 0.f;
        }
        if (l < 16) {
            // column l of the inverse of diagonal block w by forward
            // substitution, right-looking: once x[m] is final, column m of
            // the block is applied to every later x[i]. The dependent chain
            // is one FMA per row; the 15 - m updates of a step are independent.
            const int base = 16 * w;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == l) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 15; ++m)
#pragma unroll
                for (int i = m + 1; i < 16; ++i) x[i] -= sL[(base + i) * LP + base + m] * x[m];
#pragma unroll
            for (int i = 0; i < 16; ++i) sA[(base + i) * LP + base + l] = x[i];
        }
        lds_barrier();
        // Block rows: wave jb < bi forms A[bi][jb] = -A[bi][bi] T with
        // T = sum_{lb = jb}^{bi - 1} L[bi][lb] A[lb][jb], 16 x 16 blocks, on the
        // fp32 MFMA (four K = 4 steps per block product). T passes through the
        // wave's own block of sT (accumulator rows in, operand columns out).
        // A[bi][jb] replaces L[bi][jb], which the waves jb' < jb of the same
        // block row still read: it is written after the block row's barrier.
        // Every other block a wave reads is a diagonal block or a block of its
        // own column from an earlier block row, which it wrote itself.
        const int jb = w;
        float* const tb = sT + (jb < 3 ? jb : 0) * 16 * TP;  // waves 0..2 use theirs
        for (int bi = 1; bi < 4; ++bi) {
            f32x4 d = zero4();
            if (jb < bi) {
                f32x4 acc = zero4();
                for (int lb = jb; lb < bi; ++lb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4)
                        acc = mfma4(sL[(16 * bi + r) * LP + 16 * lb + 4 * q4 + g],
                                    sA[(16 * lb + 4 * q4 + g) * LP + 16 * jb + r], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) tb[(4 * g + i) * TP + r] = acc[i];
                wave_lds_sync();
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    d = mfma4(sA[(16 * bi + r) * LP + 16 * bi + 4 * q4 + g], tb[(4 * q4 + g) * TP + r], d);
            }
            lds_barrier();  // block row bi's L blocks have been read
            if (jb < bi) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sA[(16 * bi + 4 * g + i) * LP + 16 * jb + r] = -d[i];
                wave_lds_sync();
            }
        }
        // (the last block row's writes reach the other waves through the
        // barrier that closes phase 4, which touches none of sL, sA, sT)
    }

    // ---- 4. transposed operands through X * I (wave w: key / value slab w) ----
    bf16x8 ET[2][2], ZT[2][2], OT[2][2];  // [n][ks]: E^T, Z^T, dO^T frags
    {
        const bf16x8 I0 = ident_frag(0), I1 = ident_frag(1);
        // K * I: lane holds K[tok 16 mt + 4 g + e][key 32 w + 16 n + r]
        f32x4 KC[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const bf16x8 kf = tobf8(rk[mt]);
            KC[mt][0] = mfma(kf, I0, zero4());
            KC[mt][1] = mfma(kf, I1, zero4());
        }
        f32x4 EC[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int f = 32 * w + 16 * n + r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * mt + 4 * g + e;
                    EC[mt][n][e] = KC[mt][n][e] * __expf(Gat(i, f)) * (GD2 ? sEW[i * GST + f] : sBeta[i]);
                }
            }
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) ET[n][ks] = pack_pi(EC[2 * ks][n], EC[2 * ks + 1][n]);
        // V * I scaled by beta: Z^T frags of value slab w
        {
            f32x4 VC[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 vf = tobf8(rv[mt]);
                VC[mt][0] = mfma(vf, I0, zero4());
                VC[mt][1] = mfma(vf, I1, zero4());
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 16 * mt + 4 * g + e;
                        VC[mt][n][e] *= GD2 ? sEW[(CH + i) * GST + 32 * w + 16 * n + r] : sBeta[i];
                    }
            }
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) ZT[n][ks] = pack_pi(VC[2 * ks][n], VC[2 * ks + 1][n]);
        }
        if (xy) {
            f32x4 OC[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 of = tobf8(ro[mt]);
                OC[mt][0] = mfma(of, I0, zero4());
                OC[mt][1] = mfma(of, I1, zero4());
            }
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) OT[n][ks] = pack_pi(OC[2 * ks][n], OC[2 * ks + 1][n]);
        }
        if (xy || savexy) {
            // Q * I scaled by gam: Qg^T frags of key slab w
            f32x4 QC[4][2];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 qf = tobf8(rq[mt]);
                QC[mt][0] = mfma(qf, I0, zero4());
                QC[mt][1] = mfma(qf, I1, zero4());
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        QC[mt][n][e] *= __expf(Gat(16 * mt + 4 * g + e, 32 * w + 16 * n + r));
            }
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 fr = pack_pi(QC[2 * ks][n], QC[2 * ks + 1][n]);
                    const int tl = (2 * w + n) * 2 + ks;
                    if (xy) sQgT[tl * 64 + l] = fr;
                    if (savexy) st_frag(it.QgT + t * (CH * DKD), tl, fr);
                }
        }
    }
    // Kt and Qg frags (M = tok, K = key) straight from the rows
    if (walk || out) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = tid + 256 * u;
            const int i = id >> 4, f0 = (id & 15) * 8;
            float kx[8], qx[8];
            to_f8(rkr[u], kx);
            to_f8(rqr[u], qx);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float G = Gat(i, f0 + e);
                kx[e] *= __expf(Gat(CH - 1, f0 + e) - G);
                qx[e] *= __expf(G);
            }
            if (walk) st_row8_frag(it.Kt + t * (CH * DKD), i, f0, kx);
            if (out) st_row8_frag(it.Qg + t * (CH * DKD), i, f0, qx);
        }
    }
    lds_barrier();  // sQgT complete

    // ---- 5. W = A E, U = A Z; A ----
    {
        // A frag (M = tok i, K = tok j): rows 16 mt + r, cols 32 ks + pik(g, .)
        auto afrag = [&](int mt, int ks) -> bf16x8 {
            const float* row = &sA[(16 * mt + r) * LP + 32 * ks + 4 * g];
            const float4 lo = *(const float4*)row, hi = *(const float4*)(row + 16);
            const f32x4 a{lo.x, lo.y, lo.z, lo.w}, bq{hi.x, hi.y, hi.z, hi.w};
            return pack_pi(a, bq);
        };
        bf16x8 AF[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks == 0 || mt >= 2) AF[mt][ks] = afrag(mt, ks);
        if (walk) {
            // W^T (key x tok) -> -W frags (M = tok, K = key), key slab w
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 acc0 = mfma(ET[0][0], AF[mt][0], zero4());
                f32x4 acc1 = mfma(ET[1][0], AF[mt][0], zero4());
                if (mt >= 2) {
                    acc0 = mfma(ET[0][1], AF[mt][1], acc0);
                    acc1 = mfma(ET[1][1], AF[mt][1], acc1);
                }
                st_frag(it.Wn + t * (CH * DKD), mt * 4 + w, pack_pi(acc0, acc1, -1.f));
            }
        }
        if (fwdscan) {
            // U = A Z (tok x value), value slab w -> ctiles
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    f32x4 acc = mfma(AF[mt][0], ZT[n][0], zero4());
                    if (mt >= 2) acc = mfma(AF[mt][1], ZT[n][1], acc);
                    *(bf16x4*)ctile_ptr(it.U + t * (CH * DVD), (2 * w + n) * 4 + mt) = pack4(acc);
                }
        }
        if (wantA) {
            // A^T frag (M = i, K = j): slot jj of lane (r, g) = A[32 ks + pik(g, jj)][16 mt + r]
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tl = 2 * w + u, mt = tl >> 1, ks = tl & 1;
                float x[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) x[jj] = sA[(32 * ks + pik(g, jj)) * LP + 16 * mt + r];
                st_frag(it.AT + t * (CH * CH), tl, pack8(x));
            }
            if (what & PREP_AF) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int tl = 2 * w + u, mt = tl >> 1, ks = tl & 1;
                    st_frag(it.Af + t * (CH * CH), tl,
                            (ks == 0 || mt >= 2) ? afrag(mt, ks) : bf16x8{});
                }
            }
        }
    }

    // ---- 6. X = Hm^T dO, Y = Qg^T dO (value slab w) ----
    if (xy) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                f32x4 acc = zero4();
                if (mt < 2) acc = mfma(sHmT[(mt * 2 + 0) * 64 + l], OT[n][0], acc);
                acc = mfma(sHmT[(mt * 2 + 1) * 64 + l], OT[n][1], acc);
                *(bf16x4*)ctile_ptr(it.X + t * (CH * DVD), (2 * w + n) * 4 + mt) = pack4(acc);
            }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                f32x4 acc = mfma(sQgT[(mt * 2 + 0) * 64 + l], OT[n][0], zero4());
                acc = mfma(sQgT[(mt * 2 + 1) * 64 + l], OT[n][1], acc);
                *(bf16x4*)ctile_ptr(it.Y + t * (DKD * DVD), (2 * w + n) * 8 + mt) = pack4(acc);
            }
    }
}

// X = Hm^T dO, Y = Qg^T dO from stored Hm^T / Qg^T frags (full-save policy).
template <typename T>
__global__ __launch_bounds__(256, 8) void xy_kernel(Shape s, Inputs in, Inter it)
{
    ChunkRef cr;
    // the reverse walk reads chunk NC-1 first
    if (!chunk_in_order(s, blockIdx.x + (int64_t)blockIdx.y * gridDim.x, CO_ASCENDING, cr))
        return;  // an unused slot of a packed batch
    const int64_t t = cr.t;
    const int64_t tok0 = cr.tok0;  // token row of the chunk's row 0
    const int ld = (int)(s.H * DVD);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const T* dO = (const T*)in.dO + tok0 * DVD;
    const int nv = cr.nv;  // rows past it are read as zeros

    const bf16x8 I0 = ident_frag(0), I1 = ident_frag(1);
    f32x4 OC[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int i = 16 * mt + lane_r();
        float x[8];
        load8(dO + (i < nv ? i : nv - 1) * ld + 32 * w + 8 * lane_g(), x);
        const bf16x8 of = i < nv ? pack8(x) : bf16x8{};
        OC[mt][0] = mfma(of, I0, zero4());
        OC[mt][1] = mfma(of, I1, zero4());
    }
    bf16x8 OT[2][2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) OT[n][ks] = pack_pi(OC[2 * ks][n], OC[2 * ks + 1][n]);
    const bf16* HmT = it.HmT + t * (CH * CH);
    const bf16* QgT = it.QgT + t * (CH * DKD);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            f32x4 acc = zero4();
            if (mt < 2) acc = mfma(ld_frag(HmT, mt * 2 + 0), OT[n][0], acc);
            acc = mfma(ld_frag(HmT, mt * 2 + 1), OT[n][1], acc);
            *(bf16x4*)ctile_ptr(it.X + t * (CH * DVD), (2 * w + n) * 4 + mt) = pack4(acc);
        }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            f32x4 acc = mfma(ld_frag(QgT, mt * 2 + 0), OT[n][0], zero4());
            acc = mfma(ld_frag(QgT, mt * 2 + 1), OT[n][1], acc);
            *(bf16x4*)ctile_ptr(it.Y + t * (DKD * DVD), (2 * w + n) * 8 + mt) = pack4(acc);
        }
}

// A frags from the A^T frags (full-save seven-product backward; the saved
// area keeps A^T only). A frag (rows 16 rj.., K = 32 ks..) is X^T for
// X = A^T[32 ks .. + 31][16 rj .. + 15]: the two A^T tiles over rows
// 32 ks + 16 h times the identity selecting column half rj & 1 give its
// two accumulator halves, which are the frag's pik slots. Exact (each entry
// is one bf16 value times 1). One wave per (chunk, head).
__global__ __launch_bounds__(256) void a_from_at_kernel(Shape s, Inter it)
{
    ChunkRef cr;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= s.NC * (s.B * s.H)) return;
    if (!chunk_in_order(s, item, CO_DESCENDING, cr)) return;
    const bf16* AT = it.AT + cr.t * (CH * CH);
    bf16* Af = it.Af + cr.t * (CH * CH);
#pragma unroll
    for (int tl = 0; tl < 8; ++tl) {
        const int rj = tl >> 1, ks = tl & 1;
        if (ks == 1 && rj < 2) {
            st_frag(Af, tl, bf16x8{});  // above the diagonal
            continue;
        }
        const bf16x8 I = ident_pi(rj & 1);
        const f32x4 c0 = mfma(ld_frag(AT, (2 * ks) * 2 + (rj >> 1)), I, zero4());
        const f32x4 c1 = mfma(ld_frag(AT, (2 * ks + 1) * 2 + (rj >> 1)), I, zero4());
        st_frag(Af, tl, pack_pi(c0, c1));
    }
}

}  // namespace

hipError_t launch_a_from_at(const Shape& s, const Inter& it, hipStream_t st)
{
    const int64_t n = s.NC * (s.B * s.H);
    if (n <= 0) return hipSuccess;
    a_from_at_kernel<<<(unsigned)((n + 3) / 4), 256, 0, st>>>(s, it);
    return hipGetLastError();
}

hipError_t launch_prep(const Shape& s, const Inputs& in, const Inter& it, int what, hipStream_t st)
{
    dim3 grid((unsigned)s.NC, (unsigned)(s.B * s.H));
    if (s.gd2) {
        // GDN2 is built for bf16 inputs only (the host refuses the rest)
        if (s.f32 || !s.vec) return hipErrorInvalidValue;
        prep_kernel<bf16, true, true><<<grid, 256, 0, st>>>(s, in, it, what);
    } else if (s.f32) {
        if (s.vec) prep_kernel<float, true, false><<<grid, 256, 0, st>>>(s, in, it, what);
        else prep_kernel<float, false, false><<<grid, 256, 0, st>>>(s, in, it, what);
    } else {
        if (s.vec) prep_kernel<bf16, true, false><<<grid, 256, 0, st>>>(s, in, it, what);
        else prep_kernel<bf16, false, false><<<grid, 256, 0, st>>>(s, in, it, what);
    }
    return hipGetLastError();
}

hipError_t launch_xy(const Shape& s, const Inputs& in, const Inter& it, hipStream_t st)
{
    dim3 grid((unsigned)s.NC, (unsigned)(s.B * s.H));
    if (s.f32) xy_kernel<float><<<grid, 256, 0, st>>>(s, in, it);
    else xy_kernel<bf16><<<grid, 256, 0, st>>>(s, in, it);
    return hipGetLastError();
}

}  // namespace gdr
