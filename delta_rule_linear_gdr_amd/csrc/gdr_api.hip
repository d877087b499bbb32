// C ABI of the chunkwise gated delta rule (see include/gdr.h): argument
// validation, workspace carving and launch sequencing. No allocation, no
// synchronization; every launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "gdr.h"
#include "kernels.h"

namespace gdr {
namespace {

thread_local std::string g_last_error;

// Launch form of the scalar-gate three-product local backward
// (gdr_set_local_form); process-wide.
std::atomic<int> g_local_form{GDR_LOCAL_PERSISTENT};

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

constexpr size_t ALIGN = 256;
// Value widths above 128 run as 128-wide value blocks (at most 8).
constexpr int MAX_DV = 8 * DVD;
size_t align_up(size_t x) { return (x + ALIGN - 1) & ~(ALIGN - 1); }

// Per-tile byte sizes of the chunk intermediates (formats in kernels.h).
constexpr size_t B_T64x128 = CH * DKD * 2, B_T128x128 = DKD * DVD * 2, B_T64x64 = CH * CH * 2;
constexpr size_t B_GN = DKD * 4;

struct Carver {
    char* base;
    size_t off = 0;
    size_t ntiles;
    Carver(void* b, size_t n) : base((char*)b), ntiles(n) {}
    template <typename X>
    X* take(size_t per_tile)
    {
        off = align_up(off);
        X* r = base ? (X*)(base + off) : nullptr;
        off += per_tile * ntiles;
        return r;
    }
    template <typename X>
    X* take_bytes(size_t bytes)
    {
        off = align_up(off);
        X* r = base ? (X*)(base + off) : nullptr;
        off += bytes;
        return r;
    }
};

// Segments of a call's walk launch (two-level walks, scan.hip): nseg 1 is
// a one-level walk. nsh: state entries (sequences x heads).
struct WalkSeg {
    int nseg = 1;
    int64_t seglen = 0, nsh = 0;
};
// Process-wide choice of walk form (gdr_set_walk_levels): 0 automatic, 1
// always one level. The workspace is sized for the automatic form either way.
std::atomic<int> g_walk_levels{0};

// What the full-save forward keeps for the backward (its own forward scan
// reads -W and Kt from here too). A is kept once, as the A^T frags the
// three-product producer reads; the seven-product backward forms its A
// frags from them in scratch.
void carve_saved(Carver& c, Inter& it)
{
    it.AT = c.take<bf16>(B_T64x64);
    it.Kt = c.take<bf16>(B_T64x128);
    it.Wn = c.take<bf16>(B_T64x128);
    it.gn = c.take<float>(B_GN);
    it.HmT = c.take<bf16>(B_T64x64);
    it.QgT = c.take<bf16>(B_T64x128);
    it.h = c.take<bf16>(B_T128x128);
    it.R = c.take<bf16>(B_T64x128);
}

enum Phase { FWD, BWD };

// Lays out saved/scratch for one call; with null bases it only measures.
void layout(int policy, Phase ph, void* saved, void* scratch, size_t ntiles, Inter& it,
            size_t& saved_bytes, size_t& scratch_bytes, const WalkSeg& ws)
{
    memset(&it, 0, sizeof it);
    Carver sv(saved, ntiles), sc(scratch, ntiles);
    const bool full = policy == GDR_FULL_SAVE;
    // the gate-check words first, at the same place for every call and
    // policy, so that gdr_gate_status finds them from the descriptor alone
    it.flags = sc.take<uint32_t>(16);
    if (full) {
        carve_saved(sv, it);
    } else {
        // the scan operands both directions read
        it.Wn = sc.take<bf16>(B_T64x128);
        it.Kt = sc.take<bf16>(B_T64x128);
        it.gn = sc.take<float>(B_GN);
    }
    if (ph == FWD || !full) {
        // the rest of the forward scan's operands (and, in the forward, its output's)
        it.U = sc.take<bf16>(B_T64x128);
        if (ph == FWD) {
            it.Qg = sc.take<bf16>(B_T64x128);
            it.Hm = sc.take<bf16>(B_T64x64);
        }
    }
    if (ph == BWD) {
        if (!full) {
            it.AT = sc.take<bf16>(B_T64x64);
            it.Af = sc.take<bf16>(B_T64x64);
            it.h = sc.take<bf16>(B_T128x128);
            it.R = sc.take<bf16>(B_T64x128);
        }
        it.X = sc.take<bf16>(B_T64x128);
        it.Y = sc.take<bf16>(B_T128x128);
        it.dh = sc.take<bf16>(B_T128x128);
        it.Rb = sc.take<bf16>(B_T64x128);
        if (full) it.Af = sc.take<bf16>(B_T64x64);  // seven-product backward only
    }
    // two-level walks: segment summaries and entry states, both directions
    it.nseg = 1;
    it.seglen = ws.seglen;
    if (ws.nseg > 1) {
        const size_t st = (size_t)DKD * DVD * 4, nsh = (size_t)ws.nsh;
        it.seg_sum = sc.take_bytes<float>(2 * (size_t)(ws.nseg - 1) * nsh * 2 * st);
        it.seg_ent = sc.take_bytes<float>(2 * (size_t)ws.nseg * nsh * st);
        if (g_walk_levels.load(std::memory_order_relaxed) != 1) it.nseg = ws.nseg;
    }
    saved_bytes = full ? align_up(sv.off) : 0;
    scratch_bytes = align_up(sc.off);
}

__global__ void copy_or_zero(float* dst, const float* src, int64_t n)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src ? src[i] : 0.f;
}

hipError_t fill_state(float* dst, const float* src, int64_t n, hipStream_t st)
{
    if (!dst || n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    copy_or_zero<<<(unsigned)blocks, 256, 0, st>>>(dst, src, n);
    return hipGetLastError();
}

hipError_t zero_fill(float* dst, int64_t n, hipStream_t st)
{
    return fill_state(dst, nullptr, n, st);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// A packed variable-length batch (on == false: a regular batch).
struct Packed {
    bool on = false;
    const int64_t* cu = nullptr;  // device offsets, n + 1
    int64_t n = 0;                // sequences
};

int64_t nchunks(const gdr_desc* d) { return (d->T + CH - 1) / CH; }  // the last may be partial
// Chunk slots per head: all chunks of a regular row, or an upper bound on
// the chunks of the packed sequences.
int64_t nslots(const gdr_desc* d, const Packed& pk) { return nchunks(d) + (pk.on ? pk.n : 0); }
size_t ntiles(const gdr_desc* d, const Packed& pk)
{
    return (size_t)(pk.on ? d->H : d->B * d->H) * (size_t)nslots(d, pk);
}
// Two-level walks (scan.hip) replace a one-level walk launch that would fill
// at most a quarter of the chip's 256 CUs, for regular batches: the segment
// walks (a workgroup per segment and 16 value columns) and the summaries
// (twice the chains, every segment but one) must each fit one round of
// workgroups. A summary pass plus a segment walk take 2 / nseg of the
// serial steps of one walk, but each runs more workgroups at once (a step
// ~1.0 and ~0.7 us against ~0.65 for the one-level pair at (1,8192,4)), and
// chaining the entry states costs ~5 us per segment. So a segment keeps at
// least 20 chunks and there are at least 4 segments: measured at T = 8192
// with 1, 2 and 4 heads, the launches that qualify gain 11-31%, while the
// recompute pair at 3 segments, the full-save reverse walk at 4 segments of
// 16 chunks (T = 4096) and every launch at T = 2048 lose. ph / policy select
// the launch: the forward's walk, the recompute backward's two directions, or
// the full-save backward's reverse walk.
constexpr int64_t WALK_CUS = 256;
WalkSeg walk_seg(const gdr_desc* d, const Packed& pk, Phase ph, int policy)
{
    WalkSeg w;
    w.nsh = (pk.on ? pk.n : d->B) * d->H;
    if (pk.on) return w;
    const int64_t ndir = ph == BWD && policy == GDR_RECOMPUTE ? 2 : 1;
    const int64_t NT = nchunks(d), base = d->B * d->H * ndir * (DVD / 16);
    if (base <= 0 || 4 * base > WALK_CUS) return w;
    int64_t n = std::min(WALK_CUS / base, 1 + WALK_CUS / (2 * base));
    n = std::min(n, NT / 20);
    while (n > 1 && (n - 1) * ((NT + n - 1) / n) >= NT) --n;  // no empty segment
    if (n < 4) return w;
    w.nseg = (int)n;
    w.seglen = (NT + n - 1) / n;
    return w;
}

// Bytes of the sequence tables at the start of scratch (packed batches).
size_t table_bytes(const gdr_desc* d, const Packed& pk)
{
    if (!pk.on) return 0;
    return align_up(8 * (size_t)(pk.n + 1)) + align_up(8 * (size_t)pk.n) + align_up(8 * (size_t)nslots(d, pk)) +
           align_up(4 * (size_t)pk.n);
}

// DeltaNet (no decay): a zero log-decay array for the kernels and a sink for
// its gradient, after the sequence tables at the front of scratch.
bool nogate(const gdr_desc* d) { return d->gate == GDR_GATE_NONE; }
size_t gate_bytes(const gdr_desc* d) { return align_up(4 * (size_t)(d->B * d->T * d->H)); }
size_t nogate_bytes(const gdr_desc* d) { return nogate(d) ? 2 * gate_bytes(d) : 0; }

int check_desc(const gdr_desc* d)
{
    if (!d) return fail(GDR_ERR_INVALID, "descriptor is NULL");
    if (d->B < 0 || d->T < 0 || d->H < 0)
        return fail(GDR_ERR_INVALID, "negative size (B=%lld T=%lld H=%lld)", (long long)d->B,
                    (long long)d->T, (long long)d->H);
    if (d->gate != GDR_GATE_SCALAR && d->gate != GDR_GATE_VECTOR && d->gate != GDR_GATE_NONE &&
        d->gate != GDR_GATE_GDN2)
        return fail(GDR_ERR_INVALID, "unknown gate kind %d", d->gate);
    if (d->dtype != GDR_BF16 && d->dtype != GDR_F32)
        return fail(GDR_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (d->DK < 1 || d->DV < 1)
        return fail(GDR_ERR_INVALID, "key/value width %lld/%lld", (long long)d->DK, (long long)d->DV);
    if (d->DK > DKD)
        return fail(GDR_ERR_UNSUPPORTED,
                    "key width %lld: at most 128 is supported (keys couple through k k^T, so a wider key "
                    "cannot be split into 128-wide runs)",
                    (long long)d->DK);
    if (d->DV > MAX_DV)
        return fail(GDR_ERR_UNSUPPORTED, "value width %lld: at most %d is supported", (long long)d->DV, MAX_DV);
    if (d->C != CH)
        return fail(GDR_ERR_UNSUPPORTED, "chunk length %lld: only 64 is supported", (long long)d->C);
    if (d->B * d->H > 65535)
        return fail(GDR_ERR_UNSUPPORTED, "B*H=%lld exceeds 65535", (long long)(d->B * d->H));
    if ((d->T + CH - 1) / CH > (int64_t)1 << 30)
        return fail(GDR_ERR_UNSUPPORTED, "T=%lld too long", (long long)d->T);
    return GDR_OK;
}

int check_policy(int policy)
{
    if (policy != GDR_RECOMPUTE && policy != GDR_FULL_SAVE)
        return fail(GDR_ERR_INVALID, "unknown policy %d", policy);
    return GDR_OK;
}

bool gdn2(const gdr_desc* d) { return d->gate == GDR_GATE_GDN2; }

// The GDN2 entry points take the GDN2 gate kind, and only they do; GDN2 runs
// bf16 inputs.
int check_gdn2(const gdr_desc* d, bool gdn2_entry)
{
    if (gdn2(d) != gdn2_entry)
        return fail(GDR_ERR_INVALID, gdn2_entry
                                         ? "gdr_*_gdn2 takes gate kind GDR_GATE_GDN2, got %d"
                                         : "gate kind %d (GDN2) goes through gdr_fwd_gdn2 / gdr_bwd_gdn2",
                    d->gate);
    if (!gdn2_entry) return GDR_OK;
    if (d->dtype != GDR_BF16)
        return fail(GDR_ERR_UNSUPPORTED, "GDN2 is built for bf16 inputs (dtype %d)", d->dtype);
    return GDR_OK;
}

// Row tensors are read with 16-byte vector accesses; the rest element-wise.
#define REQUIRE_PTR_A(p, a)                                                            \
    do {                                                                               \
        if (!(p)) return fail(GDR_ERR_INVALID, "required pointer '%s' is NULL", #p);   \
        if ((uintptr_t)(p) % (a))                                                      \
            return fail(GDR_ERR_INVALID, "pointer '%s' is not %d-byte aligned", #p, (int)(a)); \
    } while (0)
#define REQUIRE_PTR(p) REQUIRE_PTR_A(p, 16)
#define CHECK_ALIGN(p, a)                                                              \
    do {                                                                               \
        if ((p) && (uintptr_t)(p) % (a))                                               \
            return fail(GDR_ERR_INVALID, "pointer '%s' is not %d-byte aligned", #p, (int)(a)); \
    } while (0)

Shape make_shape(const gdr_desc* d, const Packed& pk, void* scratch)
{
    Shape s;
    s.B = d->B;
    s.T = d->T;
    s.H = d->H;
    s.NT = nchunks(d);
    s.vec = d->gate == GDR_GATE_VECTOR || d->gate == GDR_GATE_GDN2;
    s.gd2 = d->gate == GDR_GATE_GDN2;
    s.f32 = d->dtype == GDR_F32;
    s.NS = pk.on ? pk.n : d->B;
    s.NC = nslots(d, pk);
    s.cu = nullptr;
    s.stab = nullptr;
    s.ctab = nullptr;
    s.order = nullptr;
    if (pk.on) {
        char* p = (char*)scratch;
        s.cu = (const int64_t*)p;
        p += align_up(8 * (size_t)(pk.n + 1));
        s.stab = (const int2*)p;
        p += align_up(8 * (size_t)pk.n);
        s.ctab = (const int2*)p;
        p += align_up(8 * (size_t)s.NC);
        s.order = (const int*)p;
    }
    return s;
}

// Validation specific to packed batches: the shape, then the offsets pointer.
int check_packed_shape(const gdr_desc* d, int64_t n_seq)
{
    if (n_seq < 0) return fail(GDR_ERR_INVALID, "negative sequence count %lld", (long long)n_seq);
    if (d->B != 1)
        return fail(GDR_ERR_INVALID, "a packed batch has B = 1 (sequences along T), got B=%lld",
                    (long long)d->B);
    if (nchunks(d) + n_seq > ((int64_t)1 << 30))
        return fail(GDR_ERR_UNSUPPORTED, "%lld sequences over T=%lld: too many chunk slots",
                    (long long)n_seq, (long long)d->T);
    if (d->T >= ((int64_t)1 << 31))  // the slot table holds 32-bit token indices
        return fail(GDR_ERR_UNSUPPORTED, "a packed row of T=%lld tokens (at most 2^31 - 1)", (long long)d->T);
    return GDR_OK;
}
int check_packed(const gdr_desc* d, const Packed& pk)
{
    int rc = check_packed_shape(d, pk.n);
    if (rc) return rc;
    if (!pk.cu) return fail(GDR_ERR_INVALID, "cu_seqlens is NULL");
    if ((uintptr_t)pk.cu % 8) return fail(GDR_ERR_INVALID, "cu_seqlens is not 8-byte aligned");
    return GDR_OK;
}

// Builds the sequence tables of a packed batch in scratch (no-op otherwise).
hipError_t seq_tables(const Shape& s, const Packed& pk, hipStream_t st)
{
    if (!pk.on) return hipSuccess;
    return launch_seq_tables(s, pk.cu, (int64_t*)s.cu, (int2*)s.stab, (int2*)s.ctab, (int*)s.order, st);
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(GDR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- optional per-stage timing (gdr_profile_begin / gdr_profile_end) ----
enum Stage {
    ST_PREP, ST_SCAN_FWD, ST_XY, ST_SCAN_BWD, ST_SCAN_PAIR, ST_BWD_LOCAL, ST_BWD_LOCAL_WY7, ST_PAD,
    ST_A_FROM_AT, NSTAGE
};
const char* const kStageName[NSTAGE] = {"prep", "scan_fwd", "xy", "scan_bwd", "scan_pair",
                                        "bwd_local", "bwd_local_wy7", "pad", "a_from_at"};

struct Profiler {
    std::mutex mu;
    bool on = false;
    bool overflow = false;
    std::vector<hipEvent_t> pool;
    struct Rec { int stage; hipEvent_t a, b; };
    std::vector<Rec> recs;
};
Profiler& prof()
{
    static Profiler p;
    return p;
}

// Runs one launch; when profiling is on, brackets it with events on `st`.
template <typename F>
hipError_t timed(Stage stage, hipStream_t st, F&& launch)
{
    Profiler& P = prof();
    std::unique_lock<std::mutex> lk(P.mu);
    if (!P.on) {
        lk.unlock();
        return launch();
    }
    if (2 * (P.recs.size() + 1) > P.pool.size()) {
        P.overflow = true;
        lk.unlock();
        return launch();
    }
    Profiler::Rec r{stage, P.pool[2 * P.recs.size()], P.pool[2 * P.recs.size() + 1]};
    hipError_t e = hipEventRecord(r.a, st);
    if (e != hipSuccess) return e;
    e = launch();
    if (e != hipSuccess) return e;
    e = hipEventRecord(r.b, st);
    if (e == hipSuccess) P.recs.push_back(r);
    return e;
}

// GDN2 gate tensors of a call (all null otherwise).
struct Gdn2Args {
    const void *ers = nullptr, *wrt = nullptr;
    void *ders = nullptr, *dwrt = nullptr;
};

int run_bwd(const gdr_desc* d, const Packed& pk, int policy, const void* q, const void* k,
            const void* v, const float* g, const void* beta, const float* h0, const void* dO,
            const float* dht, const void* saved, void* dq, void* dk, void* dv, float* dg, void* dbeta,
            float* dh0, void* scratch, size_t scratch_bytes, void* stream, bool wy7,
            const Gdn2Args& g2 = Gdn2Args{})
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    if (pk.on && (rc = check_packed(d, pk))) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t nseq = pk.on ? pk.n : d->B;
    const int64_t nstate = nseq * d->H * DKD * DVD;
    if (nseq * d->H == 0) return GDR_OK;
    if (d->T == 0) {
        hipError_t e = fill_state(dh0, dht, nstate, st);
        return e == hipSuccess ? GDR_OK : hip_fail(e, "dh0 copy");
    }
    const int esz = d->dtype == GDR_F32 ? 4 : 2;
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(dO);
    REQUIRE_PTR(dq); REQUIRE_PTR(dk); REQUIRE_PTR(dv);
    if (!nogate(d)) {
        REQUIRE_PTR_A(g, 4);
        REQUIRE_PTR_A(dg, 4);
    }
    if (gdn2(d)) {
        if (wy7) return fail(GDR_ERR_UNSUPPORTED, "GDN2 has no seven-product backward");
        const void *ers = g2.ers, *wrt = g2.wrt, *ders = g2.ders, *dwrt = g2.dwrt;
        REQUIRE_PTR(ers); REQUIRE_PTR(wrt); REQUIRE_PTR(ders); REQUIRE_PTR(dwrt);
    } else {
        REQUIRE_PTR_A(beta, esz); REQUIRE_PTR_A(dbeta, esz);
    }
    CHECK_ALIGN(h0, 4); CHECK_ALIGN(dht, 4); CHECK_ALIGN(dh0, 4);
    if (policy == GDR_FULL_SAVE) REQUIRE_PTR(saved);
    const size_t tb = table_bytes(d, pk) + nogate_bytes(d);
    Inter it;
    size_t sb = 0, need = 0;
    layout(policy, BWD, nullptr, nullptr, ntiles(d, pk), it, sb, need, walk_seg(d, pk, BWD, policy));
    need += tb;
    if (!scratch || scratch_bytes < need)
        return fail(GDR_ERR_WORKSPACE, "scratch of %zu bytes needed, %zu given", need,
                    scratch ? scratch_bytes : (size_t)0);
    if (!aligned16(scratch)) return fail(GDR_ERR_INVALID, "scratch is not 16-byte aligned");
    layout(policy, BWD, (void*)saved, (char*)scratch + tb, ntiles(d, pk), it, sb, need,
           walk_seg(d, pk, BWD, policy));

    const Shape s = make_shape(d, pk, scratch);
    hipError_t e = hipSuccess;
    if (nogate(d)) {
        float* z = (float*)((char*)scratch + table_bytes(d, pk));
        g = z;
        dg = (float*)((char*)z + gate_bytes(d));
        if ((e = zero_fill(z, d->B * d->T * d->H, st)) != hipSuccess) return hip_fail(e, "zero gate");
    }
    Inputs in{q, k, v, beta, dO, g, h0, dht, g2.ers, g2.wrt};
    Grads gr{dq, dk, dv, dbeta, dg, dh0, g2.ders, g2.dwrt};
    e = seq_tables(s, pk, st);
    if (e != hipSuccess) return hip_fail(e, "sequence tables");
    if (policy == GDR_RECOMPUTE) {
        e = timed(ST_PREP, st, [&] {
            // A itself (besides A^T) only for the seven-product producer
            return launch_prep(s, in, it, PREP_FWDSCAN | PREP_BWDSCAN | PREP_XY | PREP_A | (wy7 ? PREP_AF : 0),
                               st);
        });
        if (e != hipSuccess) return hip_fail(e, "prep");
        e = timed(ST_SCAN_PAIR, st, [&] { return launch_scan_pair(s, in, it, dh0, st); });
        if (e != hipSuccess) return hip_fail(e, "scan_pair");
    } else {
        if (wy7) {
            e = timed(ST_A_FROM_AT, st, [&] { return launch_a_from_at(s, it, st); });
            if (e != hipSuccess) return hip_fail(e, "a_from_at");
        }
        e = timed(ST_XY, st, [&] { return launch_xy(s, in, it, st); });
        if (e != hipSuccess) return hip_fail(e, "xy");
        e = timed(ST_SCAN_BWD, st, [&] { return launch_scan_bwd(s, in, it, dh0, st); });
        if (e != hipSuccess) return hip_fail(e, "scan_bwd");
    }
    // oldest in the last-level cache first: after the two walks the middle
    // chunks' h and dh; after the reverse walk alone the last chunk's dh
    const int order = policy == GDR_RECOMPUTE ? CO_MIDDLE_OUT : CO_DESCENDING;
    e = timed(wy7 ? ST_BWD_LOCAL_WY7 : ST_BWD_LOCAL, st,
              [&] {
                  return launch_bwd_local(s, in, it, gr, wy7, order,
                                          g_local_form.load() == GDR_LOCAL_PER_CHUNK, st);
              });
    if (e != hipSuccess) return hip_fail(e, "bwd_local");
    return GDR_OK;
}

int run_fwd(const gdr_desc* d, const Packed& pk, int policy, const void* q, const void* k,
            const void* v, const float* g, const void* beta, const float* h0, void* o, float* ht,
            void* saved, void* scratch, size_t scratch_bytes, void* stream,
            const Gdn2Args& g2 = Gdn2Args{})
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    if (pk.on && (rc = check_packed(d, pk))) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t nseq = pk.on ? pk.n : d->B;
    if (nseq * d->H == 0) return GDR_OK;
    if (d->T == 0) {
        hipError_t e = fill_state(ht, h0, nseq * d->H * DKD * DVD, st);
        return e == hipSuccess ? GDR_OK : hip_fail(e, "ht copy");
    }
    const int esz = d->dtype == GDR_F32 ? 4 : 2;
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(o);
    if (!nogate(d)) REQUIRE_PTR_A(g, 4);
    if (gdn2(d)) {
        const void *ers = g2.ers, *wrt = g2.wrt;
        REQUIRE_PTR(ers); REQUIRE_PTR(wrt);
    } else {
        REQUIRE_PTR_A(beta, esz);
    }
    CHECK_ALIGN(h0, 4); CHECK_ALIGN(ht, 4);
    if (policy == GDR_FULL_SAVE) REQUIRE_PTR(saved);
    const size_t tb = table_bytes(d, pk) + nogate_bytes(d);
    Inter it;
    size_t sb = 0, need = 0;
    layout(policy, FWD, nullptr, nullptr, ntiles(d, pk), it, sb, need, walk_seg(d, pk, FWD, policy));
    need += tb;
    if (!scratch || scratch_bytes < need)
        return fail(GDR_ERR_WORKSPACE, "scratch of %zu bytes needed, %zu given", need,
                    scratch ? scratch_bytes : (size_t)0);
    if (!aligned16(scratch)) return fail(GDR_ERR_INVALID, "scratch is not 16-byte aligned");
    layout(policy, FWD, saved, (char*)scratch + tb, ntiles(d, pk), it, sb, need, walk_seg(d, pk, FWD, policy));
    const Shape s = make_shape(d, pk, scratch);
    hipError_t e = hipSuccess;
    if (nogate(d)) {
        float* z = (float*)((char*)scratch + table_bytes(d, pk));
        g = z;
        if ((e = zero_fill(z, d->B * d->T * d->H, st)) != hipSuccess) return hip_fail(e, "zero gate");
    }
    Inputs in{q, k, v, beta, nullptr, g, h0, nullptr, g2.ers, g2.wrt};
    e = seq_tables(s, pk, st);
    if (e != hipSuccess) return hip_fail(e, "sequence tables");
    const int what = PREP_FWDSCAN | PREP_OUT |
                     (policy == GDR_FULL_SAVE ? PREP_BWDSCAN | PREP_SAVEXY | PREP_A : 0);
    e = timed(ST_PREP, st, [&] { return launch_prep(s, in, it, what, st); });
    if (e != hipSuccess) return hip_fail(e, "prep");
    e = timed(ST_SCAN_FWD, st, [&] { return launch_scan_fwd(s, in, it, o, ht, st); });
    if (e != hipSuccess) return hip_fail(e, "scan_fwd");
    return GDR_OK;
}


int workspace(const gdr_desc* d, const Packed& pk, int policy, size_t* saved_bytes, size_t* scratch_bytes)
{
    Inter it;
    size_t s1 = 0, c1 = 0, s2 = 0, c2 = 0;
    layout(policy, FWD, nullptr, nullptr, ntiles(d, pk), it, s1, c1, walk_seg(d, pk, FWD, policy));
    layout(policy, BWD, nullptr, nullptr, ntiles(d, pk), it, s2, c2, walk_seg(d, pk, BWD, policy));
    if (saved_bytes) *saved_bytes = s1;
    if (scratch_bytes) *scratch_bytes = table_bytes(d, pk) + nogate_bytes(d) + (c1 > c2 ? c1 : c2);
    return GDR_OK;
}

// ---- key widths below 128 and value widths other than 128: the 128-wide
//      path on zero-padded copies, one run per 128-wide value block ----
bool padded(const gdr_desc* d) { return d->DK != DKD || d->DV != DVD; }
int value_blocks(const gdr_desc* d) { return (int)((d->DV + DVD - 1) / DVD); }
gdr_desc inner_desc(const gdr_desc* d)
{
    gdr_desc e = *d;
    e.DK = DKD;
    e.DV = DVD;
    return e;
}

// The padded copies at the front of scratch (base null: sizes only).
struct PadBufs {
    void *q, *k, *v, *t4, *dq, *dk, *dv;  // token tensors, 128 wide (t4: o forward, dO backward)
    float *g, *dg;                          // vector gate and its gradient, 128 wide
    float *s0, *s1, *s2;                    // states: h0, ht or dht, dh0
    float* dg1;                             // scalar gate, value blocks after the first: dg
    void* db1;                              // value blocks after the first: dbeta
    void *ers, *wrt, *ders, *dwrt;          // GDN2 gates and their gradients, 128 wide
    size_t bytes;
};
PadBufs pad_layout(const gdr_desc* d, const Packed& pk, void* base)
{
    PadBufs p;
    memset(&p, 0, sizeof p);
    if (!padded(d)) return p;
    const size_t rows = (size_t)(d->B * d->T * d->H), esz = d->dtype == GDR_F32 ? 4 : 2;
    const size_t nst = (size_t)((pk.on ? pk.n : d->B) * d->H);
    char* b = (char*)base;
    size_t off = 0;
    auto take = [&](size_t n) -> void* {
        void* r = b ? b + off : nullptr;
        off += align_up(n);
        return r;
    };
    p.q = take(rows * DKD * esz);
    p.k = take(rows * DKD * esz);
    p.v = take(rows * DVD * esz);
    p.t4 = take(rows * DVD * esz);
    p.dq = take(rows * DKD * esz);
    p.dk = take(rows * DKD * esz);
    p.dv = take(rows * DVD * esz);
    if (d->gate == GDR_GATE_VECTOR || d->gate == GDR_GATE_GDN2) {
        p.g = (float*)take(rows * DKD * 4);
        p.dg = (float*)take(rows * DKD * 4);
    }
    if (d->gate == GDR_GATE_GDN2) {
        p.ers = take(rows * DKD * esz);
        p.wrt = take(rows * DVD * esz);
        p.ders = take(rows * DKD * esz);
        p.dwrt = take(rows * DVD * esz);
    }
    p.s0 = (float*)take(nst * DKD * DVD * 4);
    p.s1 = (float*)take(nst * DKD * DVD * 4);
    p.s2 = (float*)take(nst * DKD * DVD * 4);
    if (value_blocks(d) > 1) {
        if (d->gate == GDR_GATE_SCALAR) p.dg1 = (float*)take(rows * 4);
        if (d->gate != GDR_GATE_GDN2) p.db1 = take(rows * esz);
    }
    p.bytes = off;
    return p;
}

int workspace_any(const gdr_desc* d, const Packed& pk, int policy, size_t* saved_bytes, size_t* scratch_bytes)
{
    if (!padded(d)) return workspace(d, pk, policy, saved_bytes, scratch_bytes);
    const gdr_desc e = inner_desc(d);
    size_t sv = 0, sc = 0;
    workspace(&e, pk, policy, &sv, &sc);
    if (saved_bytes) *saved_bytes = sv * (size_t)value_blocks(d);  // one saved area per value block
    if (scratch_bytes) *scratch_bytes = pad_layout(d, pk, nullptr).bytes + sc;
    return GDR_OK;
}

// Packed batches: the device address of the sanitized offsets' last entry
// (the first token past the last sequence), which the inner call builds at
// the start of its scratch and which stays there after it; null otherwise.
const int64_t* seq_end(const Packed& pk, const void* inner_scratch)
{
    return pk.on ? (const int64_t*)inner_scratch + pk.n : nullptr;
}

// Shared checks of the padded calls; returns GDR_OK and fills pb, or a status.
int pad_prologue(const gdr_desc* d, const Packed& pk, int policy, void* scratch, size_t scratch_bytes,
                 PadBufs& pb)
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    if (pk.on && (rc = check_packed(d, pk))) return rc;
    size_t sc = 0;
    workspace_any(d, pk, policy, nullptr, &sc);
    if (!scratch || scratch_bytes < sc)
        return fail(GDR_ERR_WORKSPACE, "scratch of %zu bytes needed, %zu given", sc,
                    scratch ? scratch_bytes : (size_t)0);
    if (!aligned16(scratch)) return fail(GDR_ERR_INVALID, "scratch is not 16-byte aligned");
    pb = pad_layout(d, pk, scratch);
    return GDR_OK;
}

#define PAD_LAUNCH(expr)                                                   \
    do {                                                                   \
        hipError_t pe = timed(ST_PAD, st, [&] { return (expr); });         \
        if (pe != hipSuccess) return hip_fail(pe, "pad");                  \
    } while (0)

int run_fwd_padded(const gdr_desc* d, const Packed& pk, int policy, const void* q, const void* k,
                   const void* v, const float* g, const void* beta, const float* h0, void* o, float* ht,
                   void* saved, void* scratch, size_t scratch_bytes, void* stream, const Gdn2Args& g2)
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    if (pk.on && (rc = check_packed(d, pk))) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t nseq = pk.on ? pk.n : d->B;
    if (nseq * d->H == 0) return GDR_OK;
    if (d->T == 0) {
        hipError_t e = fill_state(ht, h0, nseq * d->H * d->DK * d->DV, st);
        return e == hipSuccess ? GDR_OK : hip_fail(e, "ht copy");
    }
    const bool g2on = gdn2(d);
    if (!q || !k || !v || !o || (g2on ? (!g2.ers || !g2.wrt) : !beta) || (!g && !nogate(d)))
        return fail(GDR_ERR_INVALID, "a required pointer is NULL");
    if (policy == GDR_FULL_SAVE && !saved) return fail(GDR_ERR_INVALID, "required pointer 'saved' is NULL");
    PadBufs pb;
    if ((rc = pad_prologue(d, pk, policy, scratch, scratch_bytes, pb))) return rc;
    const gdr_desc e = inner_desc(d);
    size_t inner_saved = 0;
    workspace(&e, pk, policy, &inner_saved, nullptr);
    const int64_t rows = d->B * d->T * d->H, nst = nseq * d->H;
    const int esz = d->dtype == GDR_F32 ? 4 : 2, dk = (int)d->DK, DV = (int)d->DV;
    const bool vec = d->gate == GDR_GATE_VECTOR || g2on;
    const int64_t* end = seq_end(pk, (char*)scratch + pb.bytes);
    const int H = (int)d->H;
    PAD_LAUNCH(launch_pad_rows(pb.q, q, rows, dk, esz, st));
    PAD_LAUNCH(launch_pad_rows(pb.k, k, rows, dk, esz, st));
    if (vec) PAD_LAUNCH(launch_pad_rows(pb.g, g, rows, dk, 4, st));
    if (g2on) PAD_LAUNCH(launch_pad_rows(pb.ers, g2.ers, rows, dk, esz, st));
    Gdn2Args gi;
    gi.ers = pb.ers;
    gi.wrt = pb.wrt;
    for (int b = 0; b < value_blocks(d); ++b) {
        // value columns [c0, c0 + dv) as their own 128-wide problem
        const int c0 = b * DVD, dv = DV - c0 < DVD ? DV - c0 : DVD;
        PAD_LAUNCH(launch_pad_rows(pb.v, v, rows, dv, esz, st, DV, c0));
        if (g2on) PAD_LAUNCH(launch_pad_rows(pb.wrt, g2.wrt, rows, dv, esz, st, DV, c0));
        if (h0) PAD_LAUNCH(launch_pad_state(pb.s0, h0, nst, dk, dv, st, DV, c0));
        rc = run_fwd(&e, pk, policy, pb.q, pb.k, pb.v, vec ? pb.g : g, beta, h0 ? pb.s0 : nullptr, pb.t4,
                     ht ? pb.s1 : nullptr, saved ? (char*)saved + b * inner_saved : nullptr,
                     (char*)scratch + pb.bytes, scratch_bytes - pb.bytes, stream, g2on ? gi : Gdn2Args{});
        if (rc) return rc;
        PAD_LAUNCH(launch_unpad_rows(o, pb.t4, rows, dv, esz, st, DV, c0, false, end, H));
        if (ht) PAD_LAUNCH(launch_unpad_state(ht, pb.s1, nst, dk, dv, st, DV, c0));
    }
    return GDR_OK;
}

int run_bwd_padded(const gdr_desc* d, const Packed& pk, int policy, const void* q, const void* k,
                   const void* v, const float* g, const void* beta, const float* h0, const void* dO,
                   const float* dht, const void* saved, void* dq, void* dk_, void* dv_, float* dg,
                   void* dbeta, float* dh0, void* scratch, size_t scratch_bytes, void* stream, bool wy7,
                   const Gdn2Args& g2)
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    if (pk.on && (rc = check_packed(d, pk))) return rc;
    hipStream_t st = (hipStream_t)stream;
    const int64_t nseq = pk.on ? pk.n : d->B;
    if (nseq * d->H == 0) return GDR_OK;
    if (d->T == 0) {
        hipError_t e = fill_state(dh0, dht, nseq * d->H * d->DK * d->DV, st);
        return e == hipSuccess ? GDR_OK : hip_fail(e, "dh0 copy");
    }
    const bool g2on = gdn2(d);
    if (!q || !k || !v || !dO || !dq || !dk_ || !dv_ || (!nogate(d) && (!g || !dg)) ||
        (g2on ? (!g2.ers || !g2.wrt || !g2.ders || !g2.dwrt) : (!beta || !dbeta)))
        return fail(GDR_ERR_INVALID, "a required pointer is NULL");
    if (g2on && wy7) return fail(GDR_ERR_UNSUPPORTED, "GDN2 has no seven-product backward");
    if (policy == GDR_FULL_SAVE && !saved) return fail(GDR_ERR_INVALID, "required pointer 'saved' is NULL");
    PadBufs pb;
    if ((rc = pad_prologue(d, pk, policy, scratch, scratch_bytes, pb))) return rc;
    const gdr_desc e = inner_desc(d);
    size_t inner_saved = 0;
    workspace(&e, pk, policy, &inner_saved, nullptr);
    const int64_t rows = d->B * d->T * d->H, nst = nseq * d->H;
    const int esz = d->dtype == GDR_F32 ? 4 : 2, dk = (int)d->DK, DV = (int)d->DV;
    const bool vec = d->gate == GDR_GATE_VECTOR || g2on, scal = d->gate == GDR_GATE_SCALAR;
    const int64_t* end = seq_end(pk, (char*)scratch + pb.bytes);
    const int H = (int)d->H;
    PAD_LAUNCH(launch_pad_rows(pb.q, q, rows, dk, esz, st));
    PAD_LAUNCH(launch_pad_rows(pb.k, k, rows, dk, esz, st));
    if (vec) PAD_LAUNCH(launch_pad_rows(pb.g, g, rows, dk, 4, st));
    if (g2on) PAD_LAUNCH(launch_pad_rows(pb.ers, g2.ers, rows, dk, esz, st));
    Gdn2Args gi;
    gi.ers = pb.ers;
    gi.wrt = pb.wrt;
    gi.ders = pb.ders;
    gi.dwrt = pb.dwrt;
    for (int b = 0; b < value_blocks(d); ++b) {
        // value columns [c0, c0 + dv) as their own 128-wide problem; the
        // key-side gradients (dq, dk, dg, dbeta) of the blocks are summed in
        // block order, the value-side ones (dv, dh0) are the block's columns
        const int c0 = b * DVD, dv = DV - c0 < DVD ? DV - c0 : DVD;
        const bool first = b == 0;
        PAD_LAUNCH(launch_pad_rows(pb.v, v, rows, dv, esz, st, DV, c0));
        PAD_LAUNCH(launch_pad_rows(pb.t4, dO, rows, dv, esz, st, DV, c0));
        if (g2on) PAD_LAUNCH(launch_pad_rows(pb.wrt, g2.wrt, rows, dv, esz, st, DV, c0));
        if (h0) PAD_LAUNCH(launch_pad_state(pb.s0, h0, nst, dk, dv, st, DV, c0));
        if (dht) PAD_LAUNCH(launch_pad_state(pb.s1, dht, nst, dk, dv, st, DV, c0));
        float* dgb = vec ? pb.dg : (scal && !first) ? pb.dg1 : dg;
        void* dbb = g2on ? nullptr : first ? dbeta : pb.db1;
        rc = run_bwd(&e, pk, policy, pb.q, pb.k, pb.v, vec ? pb.g : g, beta, h0 ? pb.s0 : nullptr, pb.t4,
                     dht ? pb.s1 : nullptr, saved ? (const char*)saved + b * inner_saved : nullptr, pb.dq, pb.dk,
                     pb.dv, dgb, dbb, dh0 ? pb.s2 : nullptr, (char*)scratch + pb.bytes, scratch_bytes - pb.bytes,
                     stream, wy7, g2on ? gi : Gdn2Args{});
        if (rc) return rc;
        if (g2on) {
            // the erase gradient is key-side (summed over the blocks), the write gradient the block's columns
            PAD_LAUNCH(launch_unpad_rows(g2.ders, pb.ders, rows, dk, esz, st, dk, 0, !first, end, H));
            PAD_LAUNCH(launch_unpad_rows(g2.dwrt, pb.dwrt, rows, dv, esz, st, DV, c0, false, end, H));
        }
        PAD_LAUNCH(launch_unpad_rows(dq, pb.dq, rows, dk, esz, st, dk, 0, !first, end, H));
        PAD_LAUNCH(launch_unpad_rows(dk_, pb.dk, rows, dk, esz, st, dk, 0, !first, end, H));
        PAD_LAUNCH(launch_unpad_rows(dv_, pb.dv, rows, dv, esz, st, DV, c0, false, end, H));
        if (vec) PAD_LAUNCH(launch_unpad_rows(dg, pb.dg, rows, dk, 4, st, dk, 0, !first, end, H));
        if (!first && !g2on) {
            // one entry per token and head: dbeta, and dg of a scalar gate
            PAD_LAUNCH(launch_add_entries(dbeta, pb.db1, rows, esz, st, end, H));
            if (scal) PAD_LAUNCH(launch_add_entries(dg, pb.dg1, rows, 4, st, end, H));
        }
        if (dh0) PAD_LAUNCH(launch_unpad_state(dh0, pb.s2, nst, dk, dv, st, DV, c0));
    }
    return GDR_OK;
}
#undef PAD_LAUNCH

// Entry dispatch: the padded path for widths other than 128. g2: the GDN2
// entry points' gate tensors (null for the beta entry points).
int any_fwd(const gdr_desc* d, const Packed& pk, int policy, const void* q, const void* k, const void* v,
            const float* g, const void* beta, const float* h0, void* o, float* ht, void* saved,
            void* scratch, size_t scratch_bytes, void* stream, const Gdn2Args* g2 = nullptr)
{
    if (!d) return check_desc(d);
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_gdn2(d, g2 != nullptr))) return rc;
    const Gdn2Args ga = g2 ? *g2 : Gdn2Args{};
    if (padded(d))
        return run_fwd_padded(d, pk, policy, q, k, v, g, beta, h0, o, ht, saved, scratch, scratch_bytes, stream,
                              ga);
    return run_fwd(d, pk, policy, q, k, v, g, beta, h0, o, ht, saved, scratch, scratch_bytes, stream, ga);
}
int any_bwd(const gdr_desc* d, const Packed& pk, int policy, const void* q, const void* k, const void* v,
            const float* g, const void* beta, const float* h0, const void* dO, const float* dht,
            const void* saved, void* dq, void* dk, void* dv, float* dg, void* dbeta, float* dh0,
            void* scratch, size_t scratch_bytes, void* stream, bool wy7, const Gdn2Args* g2 = nullptr)
{
    if (!d) return check_desc(d);
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_gdn2(d, g2 != nullptr))) return rc;
    const Gdn2Args ga = g2 ? *g2 : Gdn2Args{};
    if (padded(d))
        return run_bwd_padded(d, pk, policy, q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv, dg, dbeta, dh0,
                              scratch, scratch_bytes, stream, wy7, ga);
    return run_bwd(d, pk, policy, q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv, dg, dbeta, dh0, scratch,
                   scratch_bytes, stream, wy7, ga);
}

// ---- gate-range status (gdr_gate_status) ----
// OR of the gate-check words of every (chunk, head) in use; one workgroup.
__global__ __launch_bounds__(256) void gate_status_kernel(Shape s, const uint32_t* flags, int32_t* out)
{
    const int64_t ntile = s.NC * (s.B * s.H) * 4;
    uint32_t acc = 0;
    for (int64_t i = threadIdx.x; i < ntile; i += blockDim.x) {
        const int64_t tile = i >> 2;
        // a packed batch's unused slots were not visited by the last call
        if (s.ctab && s.ctab[tile / s.H].y <= 0) continue;
        acc |= flags[i];
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] |= red[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = (int32_t)red[0];
}

// ---- the entry point that allocates nothing (gdr_bwd_noalloc) ----
namespace noalloc {

// The workspace of gdr_bwd_noalloc: a fixed array in each device's copy of
// this code object, held from the library's load on that device to the end
// of the process. Host code never passes the array's own name to a kernel
// or a copy (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_MAX];

constexpr int MAX_DEVICES = 64;
std::mutex mu;
void* base[MAX_DEVICES];

// The array's address on device `dev` (which must be current).
int device_base(int dev, void** out)
{
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(GDR_ERR_UNSUPPORTED, "device ordinal %d (at most %d devices)", dev, MAX_DEVICES);
    std::lock_guard<std::mutex> lk(mu);
    if (!base[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(noalloc scratch)");
        if (!p || ((uintptr_t)p & 255))
            return fail(GDR_ERR_HIP, "noalloc scratch at %p is not 256-byte aligned", p);
        base[dev] = p;
    }
    *out = base[dev];
    return GDR_OK;
}

}  // namespace noalloc

}  // namespace
}  // namespace gdr

using namespace gdr;

extern "C" {

int gdr_workspace_size(const gdr_desc* d, int policy, size_t* saved_bytes, size_t* scratch_bytes)
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    return workspace_any(d, Packed{}, policy, saved_bytes, scratch_bytes);
}

int gdr_fwd(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
            const float* g, const void* beta, const float* h0, void* o, float* ht, void* saved,
            void* scratch, size_t scratch_bytes, void* stream)
{
    return any_fwd(d, Packed{}, policy, q, k, v, g, beta, h0, o, ht, saved, scratch, scratch_bytes,
                   stream);
}

int gdr_fwd_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                   const void* q, const void* k, const void* v, const float* g, const void* beta,
                   const float* h0, void* o, float* ht, void* saved, void* scratch,
                   size_t scratch_bytes, void* stream)
{
    Packed pk;
    pk.on = true;
    pk.cu = cu_seqlens;
    pk.n = n_seq;
    return any_fwd(d, pk, policy, q, k, v, g, beta, h0, o, ht, saved, scratch, scratch_bytes, stream);
}

int gdr_workspace_size_varlen(const gdr_desc* d, int64_t n_seq, int policy, size_t* saved_bytes,
                              size_t* scratch_bytes)
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    if ((rc = check_packed_shape(d, n_seq))) return rc;
    Packed pk;
    pk.on = true;
    pk.n = n_seq;
    return workspace_any(d, pk, policy, saved_bytes, scratch_bytes);
}
int gdr_bwd(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
            const float* g, const void* beta, const float* h0, const void* dO, const float* dht,
            const void* saved, void* dq, void* dk, void* dv, float* dg, void* dbeta, float* dh0,
            void* scratch, size_t scratch_bytes, void* stream)
{
    return any_bwd(d, Packed{}, policy, q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv, dg, dbeta,
                   dh0, scratch, scratch_bytes, stream, false);
}

int gdr_bwd_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                   const void* q, const void* k, const void* v, const float* g, const void* beta,
                   const float* h0, const void* dO, const float* dht, const void* saved, void* dq,
                   void* dk, void* dv, float* dg, void* dbeta, float* dh0, void* scratch,
                   size_t scratch_bytes, void* stream)
{
    Packed pk;
    pk.on = true;
    pk.cu = cu_seqlens;
    pk.n = n_seq;
    return any_bwd(d, pk, policy, q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv, dg, dbeta, dh0,
                   scratch, scratch_bytes, stream, false);
}

int gdr_bwd_noalloc(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                    const float* g, const void* beta, const float* h0, const void* dO,
                    const float* dht, const void* saved, void* dq, void* dk, void* dv, float* dg,
                    void* dbeta, float* dh0, void* stream)
{
    int rc = check_desc(d);
    if (rc) return rc;
    if ((rc = check_policy(policy))) return rc;
    size_t need = 0;
    workspace_any(d, Packed{}, policy, nullptr, &need);
    if (need > GDR_NOALLOC_SCRATCH_MAX)
        return fail(GDR_ERR_UNSUPPORTED,
                    "gdr_bwd_noalloc: this problem needs %zu bytes of scratch, more than the fixed "
                    "%zu-byte array (B*H*ceil(T/64) chunk-heads too many); use gdr_bwd with a workspace",
                    need, (size_t)GDR_NOALLOC_SCRATCH_MAX);
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if ((int)sdev != cur)
        return fail(GDR_ERR_INVALID, "gdr_bwd_noalloc: the stream belongs to device %d, device %d is current",
                    (int)sdev, cur);
    void* ws = nullptr;
    if ((rc = noalloc::device_base(cur, &ws))) return rc;
    return any_bwd(d, Packed{}, policy, q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv, dg, dbeta,
                   dh0, ws, GDR_NOALLOC_SCRATCH_MAX, stream, false);
}

int gdr_bwd_wy7(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                const float* g, const void* beta, const float* h0, const void* dO,
                const float* dht, const void* saved, void* dq, void* dk, void* dv, float* dg,
                void* dbeta, float* dh0, void* scratch, size_t scratch_bytes, void* stream)
{
    return any_bwd(d, Packed{}, policy, q, k, v, g, beta, h0, dO, dht, saved, dq, dk, dv, dg, dbeta,
                   dh0, scratch, scratch_bytes, stream, true);
}

int gdr_gate_status(const gdr_desc* d, int64_t n_seq, const void* scratch, size_t scratch_bytes,
                    int32_t* status, void* stream)
{
    int rc = check_desc(d);
    if (rc) return rc;
    Packed pk;
    if (n_seq >= 0) {
        if ((rc = check_packed_shape(d, n_seq))) return rc;
        pk.on = true;
        pk.n = n_seq;
    }
    if (!status) return fail(GDR_ERR_INVALID, "required pointer 'status' is NULL");
    if ((uintptr_t)status % 4) return fail(GDR_ERR_INVALID, "pointer 'status' is not 4-byte aligned");
    if (!scratch || !aligned16(scratch)) return fail(GDR_ERR_INVALID, "scratch is NULL or not 16-byte aligned");
    // where a call with this descriptor placed its words: after the padded
    // copies (widths below 128), then after the inner call's sequence tables
    // and DeltaNet gate arrays, first in the per-chunk layout
    const gdr_desc e = padded(d) ? inner_desc(d) : *d;
    const size_t front = (padded(d) ? pad_layout(d, pk, nullptr).bytes : 0);
    const size_t tb = table_bytes(&e, pk) + nogate_bytes(&e);
    const size_t need = front + tb + align_up(16 * ntiles(&e, pk));
    if (scratch_bytes < need)
        return fail(GDR_ERR_WORKSPACE, "scratch of %zu bytes cannot hold the gate-check words (%zu)",
                    scratch_bytes, need);
    char* inner = (char*)scratch + front;
    const Shape s = make_shape(&e, pk, inner);
    if (s.NC * (s.B * s.H) == 0) {
        hipError_t ez = zero_fill((float*)status, 1, (hipStream_t)stream);  // nothing ran: 0
        return ez == hipSuccess ? GDR_OK : hip_fail(ez, "status fill");
    }
    gate_status_kernel<<<1, 256, 0, (hipStream_t)stream>>>(s, (const uint32_t*)(inner + tb), status);
    hipError_t ee = hipGetLastError();
    return ee == hipSuccess ? GDR_OK : hip_fail(ee, "gate_status");
}

int gdr_fwd_gdn2(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                 const float* g, const void* erase, const void* write, const float* h0, void* o,
                 float* ht, void* saved, void* scratch, size_t scratch_bytes, void* stream)
{
    Gdn2Args g2;
    g2.ers = erase;
    g2.wrt = write;
    return any_fwd(d, Packed{}, policy, q, k, v, g, nullptr, h0, o, ht, saved, scratch, scratch_bytes, stream,
                   &g2);
}

int gdr_fwd_gdn2_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                        const void* q, const void* k, const void* v, const float* g, const void* erase,
                        const void* write, const float* h0, void* o, float* ht, void* saved, void* scratch,
                        size_t scratch_bytes, void* stream)
{
    Packed pk;
    pk.on = true;
    pk.cu = cu_seqlens;
    pk.n = n_seq;
    Gdn2Args g2;
    g2.ers = erase;
    g2.wrt = write;
    return any_fwd(d, pk, policy, q, k, v, g, nullptr, h0, o, ht, saved, scratch, scratch_bytes, stream, &g2);
}

int gdr_bwd_gdn2(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                 const float* g, const void* erase, const void* write, const float* h0,
                 const void* dO, const float* dht, const void* saved, void* dq, void* dk, void* dv,
                 float* dg, void* derase, void* dwrite, float* dh0, void* scratch,
                 size_t scratch_bytes, void* stream)
{
    Gdn2Args g2;
    g2.ers = erase;
    g2.wrt = write;
    g2.ders = derase;
    g2.dwrt = dwrite;
    return any_bwd(d, Packed{}, policy, q, k, v, g, nullptr, h0, dO, dht, saved, dq, dk, dv, dg, nullptr, dh0,
                   scratch, scratch_bytes, stream, false, &g2);
}

int gdr_bwd_gdn2_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                        const void* q, const void* k, const void* v, const float* g, const void* erase,
                        const void* write, const float* h0, const void* dO, const float* dht,
                        const void* saved, void* dq, void* dk, void* dv, float* dg, void* derase,
                        void* dwrite, float* dh0, void* scratch, size_t scratch_bytes, void* stream)
{
    Packed pk;
    pk.on = true;
    pk.cu = cu_seqlens;
    pk.n = n_seq;
    Gdn2Args g2;
    g2.ers = erase;
    g2.wrt = write;
    g2.ders = derase;
    g2.dwrt = dwrite;
    return any_bwd(d, pk, policy, q, k, v, g, nullptr, h0, dO, dht, saved, dq, dk, dv, dg, nullptr, dh0, scratch,
                   scratch_bytes, stream, false, &g2);
}

const char* gdr_status_string(int status)
{
    switch (status) {
    case GDR_OK: return "ok";
    case GDR_ERR_INVALID: return "invalid argument";
    case GDR_ERR_UNSUPPORTED: return "unsupported configuration";
    case GDR_ERR_WORKSPACE: return "workspace missing or too small";
    case GDR_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
    }
}

const char* gdr_last_error(void) { return g_last_error.c_str(); }

int gdr_profile_begin(int max_launches)
{
    if (max_launches < 1 || max_launches > (1 << 20))
        return fail(GDR_ERR_INVALID, "max_launches %d out of range", max_launches);
    Profiler& P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    if (P.on) return fail(GDR_ERR_INVALID, "profiling already active");
    while (P.pool.size() < 2 * (size_t)max_launches) {
        hipEvent_t ev;
        hipError_t e = hipEventCreate(&ev);
        if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
        P.pool.push_back(ev);
    }
    P.recs.clear();
    P.overflow = false;
    P.on = true;
    return GDR_OK;
}

int gdr_profile_end(gdr_stage_time* out, int cap, int* n_out)
{
    Profiler& P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    if (!P.on) return fail(GDR_ERR_INVALID, "profiling is not active");
    P.on = false;
    gdr_stage_time acc[NSTAGE];
    memset(acc, 0, sizeof acc);
    for (const auto& r : P.recs) {
        hipError_t e = hipEventSynchronize(r.b);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
        acc[r.stage].launches += 1;
        acc[r.stage].total_ms += ms;
    }
    int n = 0;
    for (int i = 0; i < NSTAGE; ++i) {
        if (acc[i].launches == 0) continue;
        if (out && n < cap) {
            out[n] = acc[i];
            snprintf(out[n].name, sizeof out[n].name, "%s", kStageName[i]);
        }
        ++n;
    }
    if (n_out) *n_out = n;
    if (P.overflow) return fail(GDR_ERR_WORKSPACE, "more launches than max_launches; tail not timed");
    return GDR_OK;
}

int gdr_set_local_form(int form)
{
    if (form != GDR_LOCAL_PERSISTENT && form != GDR_LOCAL_PER_CHUNK)
        return fail(GDR_ERR_INVALID, "unknown local-backward launch form %d", form);
    return g_local_form.exchange(form);
}

int gdr_set_walk_levels(int levels)
{
    if (levels != GDR_WALK_AUTO && levels != GDR_WALK_ONE_LEVEL)
        return fail(GDR_ERR_INVALID, "unknown walk form %d", levels);
    return g_walk_levels.exchange(levels);
}

int gdr_version(void) { return 1; }

}  // extern "C"
