// Kernel argument blocks and launch entry points of the chunkwise gated
// delta rule (gfx950). Host code in gdr_api.hip sequences these launches.
//
// Tile formats of the per-(head, chunk) intermediates. Every matrix product
// runs on v_mfma_f32_16x16x32_bf16; lane l has r = l & 15, g = l >> 4.
//
//  frag  (M x K, "contraction along K"): 16 x 32 tiles, tile (mt, ks) at
//        index mt * (K / 32) + ks, 64 lanes x 8 bf16 = 1 KiB per tile. Lane
//        (r, g) slot j holds X[16 mt + r][32 ks + pik(g, j)] with
//        pik(g, j) = 4 g + j (j < 4), 16 + 4 g + (j - 4) (j >= 4).
//        One 16-byte load per lane gives an MFMA A operand (rows of X) or B
//        operand (columns of the product = rows of X). The permuted k order
//        is the order in which two stacked 16 x 16 accumulator tiles hold
//        their rows, so an accumulator feeds the next contraction over its
//        rows without any data movement between lanes.
//  ctile (M x N): 16 x 16 accumulator tiles, tile (nt, mt) at index
//        nt * (M / 16) + mt, 64 lanes x 4 bf16 = 512 B per tile. Lane (r, g)
//        element i holds X[16 mt + 4 g + i][16 nt + r]. A column slice of
//        the matrix (fixed nt) is contiguous.
//  plain: row-major.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __bf16 bf16;

constexpr int CH = 64;    // chunk length
constexpr int DKD = 128;  // key width
constexpr int DVD = 128;  // value width

// Per-chunk intermediates; every pointer is indexed by tile t (tile_of):
// chunk-major, so the tiles of all heads for one chunk are contiguous and a
// scan step, which visits one chunk of every head, reads and writes a few
// contiguous regions rather than one region per head.
// Sizes per tile in parentheses. Unused pointers are null.
struct Inter {
    // forward scan operands (prep)
    bf16* Wn;    // -W          frag  M=64 tok,  K=128 key   (16 KiB)
    bf16* KtT;   // Kt^T        frag  M=128 key, K=64 tok    (16 KiB)
    bf16* U;     // U           ctile M=64 tok,  N=128 val   (16 KiB)
    float* gn;   // exp(G_n)    128 fp32 per key             (512 B)
    // forward output operands (prep)
    bf16* Qg;    // gam * Q     frag  M=64 tok,  K=128 key   (16 KiB)
    bf16* Hm;    // Hm          frag  M=64 tok i, K=64 tok j (8 KiB)
    // reverse scan operands (prep, xy)
    bf16* Kt;    // Kt          frag  M=64 tok,  K=128 key   (16 KiB)
    bf16* WnT;   // -W^T        frag  M=128 key, K=64 tok    (16 KiB)
    bf16* X;     // Hm^T dO     ctile M=64 tok,  N=128 val   (16 KiB)
    bf16* Y;     // Qg^T dO     ctile M=128 key, N=128 val   (32 KiB)
    bf16* HmT;   // Hm^T        frag  M=64 tok j, K=64 tok i (8 KiB)
    bf16* QgT;   // Qg^T        frag  M=128 key, K=64 tok    (16 KiB)
    // chunk-local backward inputs
    bf16* AT;    // A^T = (I+L)^-T  frag  M=64 tok i, K=64 tok j (8 KiB)
    bf16* Af;    // A             frag  M=64 tok i, K=64 tok j (8 KiB)
    bf16* h;     // state at chunk start   ctile M=128 key, N=128 val (32 KiB)
    bf16* R;     // correction             ctile M=64 tok,  N=128 val (16 KiB)
    bf16* dh;    // state adjoint at chunk end, ctile like h         (32 KiB)
    bf16* Rb;    // correction adjoint, ctile like R                 (16 KiB)
};

struct Shape {
    int64_t B, T, H, NT;
    int vec;   // 1: per-channel gate [B,T,H,128]; 0: scalar gate [B,T,H]
    int f32;   // 1: q,k,v,beta,o,dO,dq,dk,dv,dbeta are fp32; 0: bf16
};

// Tokens of chunk c: 64, except in a ragged last chunk when T % 64 != 0.
// The missing rows act as identity steps (g = 0, beta = 0, zero q, k, v and
// dO): kernels read zeros for them and write nothing for them, which leaves
// every state, output and gradient of the real tokens exact.
__host__ __device__ inline int chunk_rows(const Shape& s, int64_t c)
{
    const int64_t r = s.T - c * CH;
    return r < CH ? (int)r : CH;
}

__host__ __device__ inline int64_t tile_of(const Shape& s, int64_t bh, int64_t c)
{
    return c * (s.B * s.H) + bh;
}

struct Inputs {
    const void *q, *k, *v, *beta, *dO;
    const float *g, *h0, *dht;
};

struct Grads {
    void *dq, *dk, *dv, *dbeta;
    float *dg, *dh0;
};

// What prep writes (bit set of PREP_*).
enum {
    PREP_FWDSCAN = 1,  // Wn, KtT, U, gn
    PREP_OUT = 2,      // Qg, Hm
    PREP_BWDSCAN = 4,  // Kt, WnT (and gn)
    PREP_XY = 8,       // X, Y from dO
    PREP_SAVEXY = 16,  // HmT, QgT (for launch_xy)
    PREP_A = 32,       // AT (and Af when PREP_AF is set)
    PREP_AF = 64,
};

hipError_t launch_prep(const Shape& s, const Inputs& in, const Inter& it, int what,
                       hipStream_t st);
// X = Hm^T dO and Y = Qg^T dO from HmT, QgT and dO.
hipError_t launch_xy(const Shape& s, const Inputs& in, const Inter& it, hipStream_t st);
// Forward state scan. Writes h and R when set, the output o when o != null
// and the final state ht when ht != null.
hipError_t launch_scan_fwd(const Shape& s, const Inputs& in, const Inter& it, void* o,
                           float* ht, hipStream_t st);
// Reverse state scan (loader-fed). Writes dh and Rb (both required), and dh0
// when dh0 != null.
hipError_t launch_scan_bwd(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                           hipStream_t st);
// Both scans of the recompute backward in one loader-fed launch (the reverse
// scan does not depend on the forward one): h, R, dh, Rb (all required) and
// dh0 when dh0 != null.
hipError_t launch_scan_pair(const Shape& s, const Inputs& in, const Inter& it, float* dh0,
                            hipStream_t st);
// Chunk-local backward. wy7 selects the expanded seven-product producer.
hipError_t launch_bwd_local(const Shape& s, const Inputs& in, const Inter& it, const Grads& gr,
                            bool wy7, hipStream_t st);

}  // namespace gdr
