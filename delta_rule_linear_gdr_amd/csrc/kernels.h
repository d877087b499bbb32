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
//  ttile (M x N): a ctile's transpose within each tile, same tile order and
//        size. Lane (r, g) element i holds X[16 mt + r][16 nt + 4 g + i], so
//        the pieces of tiles (nt, mt) and (nt + 1, mt) of one lane, side by
//        side, are a frag slab of X (M = rows 16 mt.., K = columns 16 nt..
//        + 31 in pik order) with no data movement between lanes.
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
    // scan operands (prep), one orientation each: the forward scan reads
    // -W and Kt^T, the reverse scan Kt and -W^T, the transposes by LDS
    // transpose reads of the same tiles
    bf16* Wn;    // -W          frag  M=64 tok,  K=128 key   (16 KiB)
    bf16* Kt;    // Kt          frag  M=64 tok,  K=128 key   (16 KiB)
    float* gn;   // exp(G_n)    128 fp32 per key             (512 B)
    bf16* U;     // U           ctile M=64 tok,  N=128 val   (16 KiB, forward scan)
    // forward output operands (prep)
    bf16* Qg;    // gam * Q     frag  M=64 tok,  K=128 key   (16 KiB)
    bf16* Hm;    // Hm          frag  M=64 tok i, K=64 tok j (8 KiB)
    // reverse scan operands (prep, xy)
    bf16* X;     // Hm^T dO     ctile M=64 tok,  N=128 val   (16 KiB)
    bf16* Y;     // Qg^T dO     ctile M=128 key, N=128 val   (32 KiB)
    bf16* HmT;   // Hm^T        frag  M=64 tok j, K=64 tok i (8 KiB)
    bf16* QgT;   // Qg^T        frag  M=128 key, K=64 tok    (16 KiB)
    // chunk-local backward inputs
    bf16* AT;    // A^T = (I+L)^-T  frag  M=64 tok i, K=64 tok j (8 KiB)
    bf16* Af;    // A             frag  M=64 tok i, K=64 tok j (8 KiB)
    bf16* h;     // state at chunk start   ttile M=128 key, N=128 val (32 KiB)
    bf16* R;     // correction             ttile M=64 tok,  N=128 val (16 KiB)
    bf16* dh;    // state adjoint at chunk end, ttile like h         (32 KiB)
    bf16* Rb;    // correction adjoint     ctile M=64 tok,  N=128 val (16 KiB)
    // gate check (prep): one word per prep wave, OR of GATE_* bits   (16 B)
    uint32_t* flags;
    // Two-level walks (regular batches whose one-level walks would leave
    // most CUs idle): each walk is cut into nseg segments of seglen chunks
    // (the last may be shorter). Per direction d (0 forward, 1 reverse):
    //   seg_sum [d][nseg - 1][B*H][2][128][128] fp32: a segment's transfer
    //           map Phi (entry state -> exit state, keys x keys), then its
    //           exit state from a zero entry state E (keys x values), for
    //           every segment but the last in walk order (index: the
    //           segment's position among those);
    //   seg_ent [d][nseg][B*H][128][128] fp32: each segment's entry state.
    int nseg;        // 1: one serial walk
    int64_t seglen;
    float* seg_sum;
    float* seg_ent;
};

// Gate-check bits prep records per (chunk, head) (gdr_gate_status).
enum {
    GATE_POSITIVE = 1,   // a log decay above 0 (not a decay)
    GATE_RANGE = 2,      // vector gate: a 16-token window's per-key range above GATE_RANGE_MAX
    GATE_NONFINITE = 4,  // a log decay that is NaN or infinite
};
constexpr float GATE_RANGE_MAX = 160.f;

struct Shape {
    int64_t B, T, H, NT;
    int vec;   // 1: per-channel gate [B,T,H,128]; 0: scalar gate [B,T,H]
    int f32;   // 1: q,k,v,beta,o,dO,dq,dk,dv,dbeta are fp32; 0: bf16
    int gd2;   // 1: GDN2 -- per-channel gate with independent erase and write
               // gates (Inputs::ers, wrt; Grads::ders, dwrt) in place of beta
    // Sequences (state entries) and chunk slots per head. Regular batch:
    // NS = B, NC = NT. Packed variable-length batch (B = 1): NS sequences,
    // NC = ceil(T / 64) + NS (at least the chunks of all sequences) and the
    // device tables below, null otherwise.
    int64_t NS, NC;
    const int64_t* cu;  // sanitized token offsets, NS + 1
    const int2* stab;   // per sequence: {first chunk slot, chunk count}
    const int2* ctab;   // per chunk slot: {token (along T) of its row 0, rows}, rows 0 if unused
    const int* order;   // sequences, longest first (by length class), for the scans
};

// One sequence of one head. Each sequence is chunked on its own; its last
// chunk may be ragged. The missing rows of a ragged chunk act as identity
// steps (g = 0, beta = 0, zero q, k, v and dO): kernels read zeros for them
// and write nothing for them, which leaves every state, output and gradient
// of the real tokens exact.
struct SeqView {
    int64_t tok;     // token index (along T) of the sequence's first token
    int64_t len;     // its tokens
    int64_t nchunk;  // its chunks (a segment view: the segment's)
    int64_t slot0;   // chunk slot of its chunk 0 (packed batches)
    int64_t n, hd;   // sequence (state entry) and head
    int64_t c0;      // chunk 0 of the view within the sequence (a segment of a walk)
};

__host__ __device__ inline SeqView seq_view(const Shape& s, int64_t n, int64_t hd)
{
    SeqView v;
    v.n = n;
    v.hd = hd;
    if (s.ctab) {
        v.tok = s.cu[n];
        v.len = s.cu[n + 1] - v.tok;
        v.slot0 = s.stab[n].x;
        v.nchunk = s.stab[n].y;
    } else {
        v.tok = n * s.T;
        v.len = s.T;
        v.slot0 = 0;
        v.nchunk = s.NT;
    }
    v.c0 = 0;
    return v;
}

// Chunks [c0, c0 + n) of a sequence view, seen as a sequence of their own.
__host__ __device__ inline SeqView seg_view(SeqView v, int64_t c0, int64_t n)
{
    v.c0 += c0;
    v.nchunk = n;
    return v;
}

// Tile index of chunk c: chunk-major, so the tiles of all heads for one
// chunk (slot) are contiguous and a scan step, which visits one chunk of
// every head, reads and writes a few contiguous regions.
__host__ __device__ inline int64_t seq_tile(const Shape& s, const SeqView& v, int64_t c)
{
    c += v.c0;
    return s.ctab ? (v.slot0 + c) * s.H + v.hd : c * (s.B * s.H) + v.n * s.H + v.hd;
}

// Valid rows of chunk c (64 except in a ragged last chunk).
__host__ __device__ inline int seq_rows(const SeqView& v, int64_t c)
{
    const int64_t r = v.len - (v.c0 + c) * CH;
    return r < CH ? (int)r : CH;
}

// Row index into [.., T, H, ..] token-major tensors of chunk c's first token.
__host__ __device__ inline int64_t seq_tok0(const Shape& s, const SeqView& v, int64_t c)
{
    return (v.tok + (v.c0 + c) * CH) * s.H + v.hd;
}

// What a per-chunk kernel needs of its (chunk, head): the tile, the row
// index (into [.., T, H, ..] token-major tensors) of the chunk's first token,
// and its rows (past them: zeros read, nothing written).
struct ChunkRef {
    int64_t t, tok0;
    int nv;
};

// The chunk at (x = chunk or chunk slot, y = b * H + head), as seq_tile,
// seq_tok0 and seq_rows give it for the sequence view of (b, head); in a
// packed batch from the slot's table entry alone (one read), false for an
// unused slot.
__device__ inline bool chunk_at(const Shape& s, int64_t x, int64_t y, ChunkRef& r)
{
    if (s.ctab) {
        const int2 e = s.ctab[x];
        if (e.y <= 0) return false;
        r.t = x * s.H + y;
        r.tok0 = (int64_t)e.x * s.H + y;
        r.nv = e.y;
    } else {
        const SeqView v = seq_view(s, y / s.H, y % s.H);
        r.t = seq_tile(s, v, x);
        r.tok0 = seq_tok0(s, v, x);
        r.nv = seq_rows(v, x);
    }
    return true;
}

// Order in which a launch over the (chunk, head) pairs of a regular batch
// visits them. The chip's 256 MiB last-level cache keeps the most recently
// written intermediates, so a producer visits the chunks chunk-major (every
// head of one chunk in turn) and writes last what its consumer reads first:
//   CO_ASCENDING   0 .. NC-1 (for a consumer walking NC-1 .. 0),
//   CO_DESCENDING  NC-1 .. 0 (for a consumer walking 0 .. NC-1),
//   CO_MIDDLE_OUT  the middle chunks first and both ends last (for the
//                  forward and reverse walks run side by side).
// A consumer of the walks' own outputs visits first what is oldest in the
// cache, before the new traffic evicts it.
enum ChunkOrder { CO_ASCENDING = 0, CO_DESCENDING = 1, CO_MIDDLE_OUT = 2 };

__device__ inline int64_t ordered_chunk(int64_t k, int64_t NC, int order)
{
    if (order == CO_ASCENDING) return k;
    if (order == CO_DESCENDING) return NC - 1 - k;
    const int64_t mid = (NC - 1) / 2;  // k = 0, 1, 2, 3, ... -> mid, mid + 1, mid - 1, mid + 2, ...
    return (k & 1) ? mid + 1 + k / 2 : mid - k / 2;
}

// Chunk slots in use: NC in a regular batch; in a packed batch the
// sequences' slots, which are 0 .. U-1 (each sequence's first slot is the
// exclusive sum of the chunk counts before it), the rest of NC unused.
__device__ inline int64_t slots_used(const Shape& s)
{
    if (!s.ctab) return s.NC;
    if (s.NS <= 0) return 0;
    const int2 e = s.stab[s.NS - 1];
    return (int64_t)e.x + e.y;
}

// Item L (0 .. NC * B * H - 1) of a launch: the (chunk, b * H + head) pair
// at position L of `order` over the slots in use (in a packed batch, B = 1,
// the order runs over the chunk slots, sequence after sequence); items past
// them yield false. Either way the concurrent workgroups of a launch touch
// neighbouring tiles (tiles are chunk- or slot-major).
// NU: slots_used(s), which a caller mapping many items reads once.
__device__ inline bool chunk_in_order(const Shape& s, int64_t L, int order, int64_t NU, ChunkRef& r)
{
    const int64_t BH = s.B * s.H, k = L / BH;
    if (k >= NU) return false;
    return chunk_at(s, ordered_chunk(k, NU, order), L % BH, r);
}
__device__ inline bool chunk_in_order(const Shape& s, int64_t L, int order, ChunkRef& r)
{
    return chunk_in_order(s, L, order, slots_used(s), r);
}

// Compute units of the current device (cached per device).
int cu_count();

struct Inputs {
    const void *q, *k, *v, *beta, *dO;
    const float *g, *h0, *dht;
    // GDN2: erase gate [B,T,H,128] (per key) and write gate [B,T,H,128]
    // (per value), bf16; null otherwise
    const void *ers, *wrt;
};

struct Grads {
    void *dq, *dk, *dv, *dbeta;
    float *dg, *dh0;
    void *ders, *dwrt;  // GDN2: gradients of the erase and write gates
};

// What prep writes (bit set of PREP_*).
enum {
    PREP_FWDSCAN = 1,  // Wn, Kt, gn and U
    PREP_OUT = 2,      // Qg, Hm
    PREP_BWDSCAN = 4,  // Wn, Kt, gn
    PREP_XY = 8,       // X, Y from dO
    PREP_SAVEXY = 16,  // HmT, QgT (for launch_xy)
    PREP_A = 32,       // AT (and Af when PREP_AF is set)
    PREP_AF = 64,
};

hipError_t launch_prep(const Shape& s, const Inputs& in, const Inter& it, int what,
                       hipStream_t st);
// A frags (it.Af) from the A^T frags (it.AT), every (chunk, head): what the
// full-save seven-product backward needs, the saved area holding A^T only.
hipError_t launch_a_from_at(const Shape& s, const Inter& it, hipStream_t st);
// X = Hm^T dO and Y = Qg^T dO from HmT, QgT and dO.
hipError_t launch_xy(const Shape& s, const Inputs& in, const Inter& it, hipStream_t st);
// Forward state scan (loader-fed; its loader waves also form the output).
// Writes the output o (required), h and R when it.h is set, and the final
// state ht when ht != null.
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
// Packed batches: sanitizes cu_in (clamped to [0, T], made nondecreasing)
// into s.cu and fills s.stab, s.ctab and s.order (one workgroup).
hipError_t launch_seq_tables(const Shape& s, const int64_t* cu_in, int64_t* cu, int2* stab, int2* ctab,
                             int* order, hipStream_t st);
// Widths other than 128 (pad.hip): rows of width w <-> rows of width 128
// (zeros past w), esz = element bytes; states [n][dk][dv] <-> [n][128][128].
// The wide side may be a column block: ld = its row length (0: w), col0 =
// the block's first column; add = accumulate into dst (type from esz).
hipError_t launch_pad_rows(void* dst, const void* src, int64_t rows, int w, int esz, hipStream_t st,
                           int src_ld = 0, int col0 = 0);
// end: null, or (packed batches) the device address of the first token past
// the last sequence; rows from token *end on (per rows a token) are skipped
hipError_t launch_unpad_rows(void* dst, const void* src, int64_t rows, int w, int esz, hipStream_t st,
                             int dst_ld = 0, int col0 = 0, bool add = false, const int64_t* end = nullptr,
                             int per = 1);
hipError_t launch_pad_state(float* dst, const float* src, int64_t n, int dk, int dv, hipStream_t st,
                            int src_dv = 0, int col0 = 0);
// dst[i] += src[i] for n entries of esz bytes (bf16 or fp32)
hipError_t launch_add_entries(void* dst, const void* src, int64_t n, int esz, hipStream_t st,
                              const int64_t* end = nullptr, int per = 1);
hipError_t launch_unpad_state(float* dst, const float* src, int64_t n, int dk, int dv, hipStream_t st,
                              int dst_dv = 0, int col0 = 0);
// Chunk-local backward. wy7 selects the expanded seven-product producer.
// order: the ChunkOrder of the (chunk, head) items (regular batches).
// per_chunk: launch the scalar-gate three-product kernel one workgroup per
// (chunk, head), like the other local kernels, instead of its persistent
// form (same results; for like-for-like timing against the seven-product one).
hipError_t launch_bwd_local(const Shape& s, const Inputs& in, const Inter& it, const Grads& gr,
                            bool wy7, int order, bool per_chunk, hipStream_t st);

}  // namespace gdr
