// Device helpers shared by the gfx950 kernels of the chunkwise gated delta rule.
//
// Matrix products use v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulation). Operand fragments follow the instruction's lane layout:
//   A (16 x 32, M x K):  lane l holds row (l & 15), k = 8*(l >> 4) .. +7
//   B (32 x 16, K x N):  lane l holds col (l & 15), k = 8*(l >> 4) .. +7
//   C (16 x 16):         lane l holds col (l & 15), rows 4*(l >> 4) .. +3
// Both operands are therefore read from "K-contiguous" storage: A as [M][K]
// and B transposed as Bt[N][K], one 16-byte read per lane per fragment.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace gdr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS row strides (elements): 16 bytes of padding per row spreads the rows of
// one fragment read over distinct banks.
constexpr int LD128 = DKD + 8;  // rows of 128 bf16
constexpr int LD64 = CH + 8;    // rows of 64 bf16

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// K = 16 product, v_mfma_f32_16x16x16_bf16: lane l holds A row (l & 15) (or B
// column (l & 15)) at k = 4 (l >> 4) .. + 3; the accumulator layout is that of
// the K = 32 product. Either half of a pik-ordered frag (below) is such an
// operand: elements 0..3 carry k-slots 0..15 of the 32, elements 4..7 k-slots
// 16..31, each in natural order.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                     c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Storage element types of the operator's inputs/outputs.
template <typename T> struct io;
template <> struct io<bf16> {
    __device__ static float ld(const bf16* p) { return (float)*p; }
    __device__ static void st(bf16* p, float x) { *p = (bf16)x; }
};
template <> struct io<float> {
    __device__ static float ld(const float* p) { return *p; }
    __device__ static void st(float* p, float x) { *p = x; }
};

// Load 8 consecutive elements of an input row as floats.
__device__ __forceinline__ void load8(const bf16* p, float (&x)[8])
{
    bf16x8 v = *(const bf16x8*)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8])
{
    float4 a = *(const float4*)p;
    float4 b = *(const float4*)(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8])
{
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    *(bf16x8*)p = v;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8])
{
    *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
    *(float4*)(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ __forceinline__ bf16x8 pack8(const float (&x)[8])
{
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    return v;
}

// Fragment reads (LDS or global), K-contiguous storage with row stride ld.
__device__ __forceinline__ bf16x8 frag(const bf16* base, int ld, int row0, int k0)
{
    const int l = lane_id();
    return *(const bf16x8*)(base + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
}

// acc[mt][nt] += A[m0+16mt.., k] * Bt[n0+16nt.., k] for k in [0, K).
template <int MT, int NT, int K>
__device__ __forceinline__ void wave_gemm(const bf16* A, int lda, int m0, const bf16* Bt, int ldb,
                                          int n0, f32x4 (&acc)[MT][NT])
{
#pragma unroll
    for (int k = 0; k < K; k += 32) {
        bf16x8 a[MT], b[NT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) a[mt] = frag(A, lda, m0 + 16 * mt, k);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) b[nt] = frag(Bt, ldb, n0 + 16 * nt, k);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma(a[mt], b[nt], acc[mt][nt]);
    }
}

// Row/column of element r of a C fragment whose tile origin is (m0, n0).
__device__ __forceinline__ int crow(int m0, int r) { return m0 + 4 * (lane_id() >> 4) + r; }
__device__ __forceinline__ int ccol(int n0) { return n0 + (lane_id() & 15); }

// Write a C fragment into a row-major bf16 buffer: buf[row][col].
__device__ __forceinline__ void put_c(bf16* buf, int ld, int m0, int n0, const f32x4& c,
                                      float scale = 1.f)
{
    const int col = ccol(n0);
#pragma unroll
    for (int r = 0; r < 4; ++r) buf[crow(m0, r) * ld + col] = (bf16)(c[r] * scale);
}
// Write a C fragment transposed: buf[col][row .. row+3] (one 8-byte write).
__device__ __forceinline__ void put_c_t(bf16* buf, int ld, int m0, int n0, const f32x4& c,
                                        float scale = 1.f)
{
    bf16x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (bf16)(c[r] * scale);
    *(bf16x4*)(buf + ccol(n0) * ld + crow(m0, 0)) = v;
}

// ---------------------------------------------------------------- cross-lane
// Register-only exchanges (no LDS round trip): DPP row rotations inside a
// 16-lane row, and the gfx950 permlane swaps between rows.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes that share (lane >> 4), i.e. over the columns of a C
// fragment row group; every lane of the row receives a sum (row rotations
// by 8, 4, 2, 1).
__device__ __forceinline__ float sum16(float x)
{
    x += dpp_f<0x128>(x);
    x += dpp_f<0x124>(x);
    x += dpp_f<0x122>(x);
    x += dpp_f<0x121>(x);
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: scans inside each
// 16-lane row (row shifts by 1, 2, 4, 8), then the last lane of a row is
// added to the next row (row_bcast:15, rows 1 and 3) and lane 31 to rows 2
// and 3 (row_bcast:31). Lanes a shift does not reach add zero.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_zero(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_incl_scan(float x)
{
    x += dpp_zero<0x111, 0xf>(x);
    x += dpp_zero<0x112, 0xf>(x);
    x += dpp_zero<0x114, 0xf>(x);
    x += dpp_zero<0x118, 0xf>(x);
    x += dpp_zero<0x142, 0xa>(x);
    x += dpp_zero<0x143, 0xc>(x);
    return x;
}

// Inclusive suffix sum over the 64 lanes of a wave (lane l receives the
// sum over lanes l .. 63): suffix sums inside each 16-lane row (row shifts
// left by 1, 2, 4, 8), then the totals of the later rows, read from their
// first lanes.
__device__ __forceinline__ float wave_incl_suffix(float x)
{
    x += dpp_zero<0x101, 0xf>(x);
    x += dpp_zero<0x102, 0xf>(x);
    x += dpp_zero<0x104, 0xf>(x);
    x += dpp_zero<0x108, 0xf>(x);
    const float t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float t2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float t3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    const int row = lane_id() >> 4;
    return x + (row < 3 ? t3 : 0.f) + (row < 2 ? t2 : 0.f) + (row < 1 ? t1 : 0.f);
}

// Value held by lane l ^ 16 (rows 0 <-> 1, 2 <-> 3) and by lane l ^ 32.
// A swap returns this lane's own value in one result and the partner's in
// the other; comparing bits picks the partner's (if both are equal, either
// is right). Call these as plain statements, never as an operand of ?: or
// under a lane-dependent branch: a swap issued with some lanes masked off
// does not receive those lanes' values.
__device__ __forceinline__ float partner16(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(p[0] == u ? p[1] : p[0]);
}
__device__ __forceinline__ float partner32(float x)
{
    const unsigned u = __float_as_uint(x);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(p[0] == u ? p[1] : p[0]);
}
// x summed over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four rows); the
// same value in all four (addition is commutative).
__device__ __forceinline__ float sum_rows(float x)
{
    x += partner16(x);
    return x + partner32(x);
}


// ---------------------------------------------------------------- tile formats
// (see kernels.h for the frag and ctile formats)

__device__ __forceinline__ int lane_r() { return threadIdx.x & 15; }
__device__ __forceinline__ int lane_g() { return (threadIdx.x >> 4) & 3; }

// k offset inside a 32-wide slab of slot j held by lane group g.
__host__ __device__ __forceinline__ int pik(int g, int j) { return j < 4 ? 4 * g + j : 12 + 4 * g + j; }

// Two accumulator tiles stacked along M (rows 0..15 in lo, 16..31 in hi)
// as one frag slab: slots 0..3 from lo, 4..7 from hi.
__device__ __forceinline__ bf16x8 pack_pi(const f32x4& lo, const f32x4& hi, float s = 1.f)
{
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = (bf16)(lo[i] * s);
        v[4 + i] = (bf16)(hi[i] * s);
    }
    return v;
}
__device__ __forceinline__ bf16x4 pack4(const f32x4& c, float s = 1.f)
{
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)(c[i] * s);
    return v;
}
__device__ __forceinline__ f32x4 unpack4(const bf16x4& v)
{
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}

// Lane pointer into frag tile `tile` of a buffer.
__device__ __forceinline__ bf16* frag_ptr(bf16* base, int tile) { return base + (tile * 64 + lane_id()) * 8; }
__device__ __forceinline__ const bf16* frag_ptr(const bf16* base, int tile)
{
    return base + (tile * 64 + lane_id()) * 8;
}
__device__ __forceinline__ bf16x8 ld_frag(const bf16* base, int tile) { return *(const bf16x8*)frag_ptr(base, tile); }
__device__ __forceinline__ void st_frag(bf16* base, int tile, const bf16x8& v) { *(bf16x8*)frag_ptr(base, tile) = v; }
// Where slot s (the 16 bytes of lane s) of a frag tile sits in an LDS copy
// read by ld_frag_t64x128: s ^ 4 (s >> 4). An involution; a plain read of
// the copy by lane l at this position stays conflict-free, and the
// transposed read below hits 16 distinct bank pairs per 16 lanes instead of
// 4 (unpermuted, the four key groups of one row lie 256 bytes apart).
__host__ __device__ __forceinline__ int tr_slot(int s) { return s ^ ((s >> 2) & 12); }

// Frag tile (mt, ks) of X^T read from X's own frag tiles in LDS, X being
// M x K with K / 32 = 4 (M = 64 tokens, K = 128 keys; X^T is 128 x 64, so
// mt < 8 and ks < 2). Uses gfx950's transposing LDS read (ds_read_b64_tr_b16):
// within each group of 16 lanes, lane j receives as element e the element
// j & 3 of what lane 4 e + (j >> 2) loaded. So lane (r, g) of the group g
// loads, for the first half of its fragment, 8 bytes of token row
// R = 32 ks + 4 g + (r >> 2) (the second half: R + 16) -- keys
// 16 mt + 4 (r & 3) .. + 3, which X's frag tile (R / 16, mt / 2) holds
// contiguously in slot half mt & 1 of lane (R & 15) + 16 (r & 3) -- and
// receives X[32 ks + pik(g, j)][16 mt + r], slot j, as the frag format asks.
// xs: the LDS base of X's 16 frag tiles (1 KiB each, tile (m, k) at m * 4 + k),
// their slots placed by tr_slot.
__device__ __forceinline__ bf16x8 ld_frag_t64x128(const uint8_t* xs, int mt, int ks)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int r = lane_id() & 15, g = lane_id() >> 4;
    const int slot = tr_slot(4 * g + (r >> 2) + 16 * (r & 3));
    const uint8_t* p = xs + (2 * ks * 4 + (mt >> 1)) * 1024 + slot * 16 + 8 * (mt & 1);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 4 * 1024));
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// The same for X 64 x 64 (K / 32 = 2: frag tiles (m, k) at m * 2 + k, 8 KiB;
// X^T is 64 x 64, mt < 4 and ks < 2).
__device__ __forceinline__ bf16x8 ld_frag_t64x64(const bf16x8* xs, int mt, int ks)
{
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int r = lane_id() & 15, g = lane_id() >> 4;
    const int slot = tr_slot(4 * g + (r >> 2) + 16 * (r & 3));
    const uint8_t* p = (const uint8_t*)xs + (2 * ks * 2 + (mt >> 1)) * 1024 + slot * 16 + 8 * (mt & 1);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 2 * 1024));
    const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
    return __builtin_shufflevector(l4, h4, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Lane pointer into ctile `tile`.
__device__ __forceinline__ const bf16* ctile_ptr(const bf16* base, int tile)
{
    return base + (tile * 64 + lane_id()) * 4;
}
__device__ __forceinline__ bf16* ctile_ptr(bf16* base, int tile) { return base + (tile * 64 + lane_id()) * 4; }

// B operand of X * I for output column tile nt: the identity restricted to
// k slab nt >> 1 (the other slabs are zero). parity = nt & 1.
// (`lane` lets a caller pass a lane index the compiler cannot hoist.)
__device__ __forceinline__ bf16x8 ident_frag(int parity, int lane)
{
    const int r = lane & 15, g = (lane >> 4) & 3;
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16)((8 * g + j == 16 * parity + r) ? 1.f : 0.f);
    return v;
}
__device__ __forceinline__ bf16x8 ident_frag(int parity) { return ident_frag(parity, lane_id()); }

// The same identity for an A operand in frag (pik) k order, e.g. one
// assembled from accumulator tiles: slot j is 1 where pik(g, j) is the
// output column.
__device__ __forceinline__ bf16x8 ident_pi(int parity, int lane)
{
    const int r = lane & 15, g = (lane >> 4) & 3;
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (bf16)((pik(g, j) == 16 * parity + r) ? 1.f : 0.f);
    return v;
}
__device__ __forceinline__ bf16x8 ident_pi(int parity) { return ident_pi(parity, lane_id()); }

__device__ __forceinline__ bf16x8 cat8(const bf16x4& lo, const bf16x4& hi)
{
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = lo[i];
        v[4 + i] = hi[i];
    }
    return v;
}
// The halves of a pik-ordered frag as K = 16 operands (k-slots 0..15 and 16..31).
__device__ __forceinline__ bf16x4 half0(const bf16x8& v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 half1(const bf16x8& v) { return __builtin_shufflevector(v, v, 4, 5, 6, 7); }

// Four consecutive elements of an input/output row.
__device__ __forceinline__ void load4(const bf16* p, float (&x)[4])
{
    const bf16x4 v = *(const bf16x4*)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load4(const float* p, float (&x)[4])
{
    const float4 v = *(const float4*)p;
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void store4(bf16* p, const float (&x)[4])
{
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
    *(bf16x4*)p = v;
}
__device__ __forceinline__ void store4(float* p, const float (&x)[4])
{
    *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
}
// The same as a streaming (non-temporal) store, for results that no later
// access of the same launch reads: they then leave the L2 to the operand
// tiles the launch's workgroups share.
__device__ __forceinline__ void store4_stream(bf16* p, const float (&x)[4])
{
    bf16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)x[e];
    __builtin_nontemporal_store(v, (bf16x4*)p);
}
__device__ __forceinline__ void store4_stream(float* p, const float (&x)[4])
{
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, (f32x4*)p);
}

// Workgroup barrier for an LDS exchange only. __syncthreads() also orders
// global memory, so it waits for every outstanding global load and store of
// the wave (a full vmcnt(0)); these kernels never read back global data that
// another wave of the workgroup wrote, so the barrier waits only for the
// wave's LDS accesses and leaves its loads in flight and its stores
// draining. (The inline s_barrier carries no implied waits; the clobber
// keeps memory accesses on their side of it.)
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0); vmcnt, expcnt at their maxima
    asm volatile("s_barrier" ::: "memory");
}

// Orders a wave's LDS writes before its later LDS reads of data that other
// lanes of the same wave wrote. The LDS serves one wave's accesses in issue
// order, so only the compiler's order has to be held (the memory clobber);
// the wait also completes the writes before any later read is issued.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// fp32 product C += A B with A 16 x 4 and B 4 x 16 (v_mfma_f32_16x16x4_f32):
// lane (r, g) passes A[r][g] and B[g][r]; accumulator element i of lane
// (r, g) is C[4 g + i][r], as for the bf16 products.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Cache-policy operand of the load builtins for a streaming ("nt") access.
constexpr int CPOL_NT = 2;

// Direct-to-LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane L
// reads src and its bytes land at lds_base + 16 L; lds_base must be the
// same for every lane. Completion is counted by the vector-memory counter.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds_base)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Unconverted reads of 4 and 8 consecutive elements, so that a batch of
// reads can be issued before the first of them is consumed.
struct f32x8 {
    f32x4 a, b;
};
__device__ __forceinline__ bf16x4 ld4raw(const bf16* p) { return *(const bf16x4*)p; }
__device__ __forceinline__ f32x4 ld4raw(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ bf16x8 ld8raw(const bf16* p) { return *(const bf16x8*)p; }
__device__ __forceinline__ f32x8 ld8raw(const float* p)
{
    return f32x8{*(const f32x4*)p, *(const f32x4*)(p + 4)};
}
__device__ __forceinline__ f32x4 tof4(const bf16x4& v) { return unpack4(v); }
__device__ __forceinline__ f32x4 tof4(const f32x4& v) { return v; }
__device__ __forceinline__ bf16x4 tobf4(const bf16x4& v) { return v; }
__device__ __forceinline__ bf16x4 tobf4(const f32x4& v) { return pack4(v); }
__device__ __forceinline__ bf16x8 tobf8(const bf16x8& v) { return v; }
__device__ __forceinline__ bf16x8 tobf8(const f32x8& v) { return cat8(pack4(v.a), pack4(v.b)); }

__device__ __forceinline__ void to_f8(const bf16x8& v, float (&x)[8])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void to_f8(const f32x8& v, float (&x)[8])
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = v.a[e];
        x[4 + e] = v.b[e];
    }
}

// Plain-order fragment of a row-major matrix with row stride ld (elements):
// lane (r, g) gets X[row0 + r][k0 + 8 g .. + 7] as floats.
template <typename T>
__device__ __forceinline__ void ld_plain8(const T* base, int ld, int row0, int k0, float (&x)[8])
{
    load8(base + (row0 + lane_r()) * ld + k0 + 8 * lane_g(), x);
}

}  // namespace gdr
