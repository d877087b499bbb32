/*
 * gdr.h -- C ABI of the MI355X (gfx950) chunkwise gated delta-rule operator:
 * forward and backward of Gated DeltaNet (scalar gate), Kimi Delta
 * Attention (per-key-channel gate), DeltaNet (no decay) and GDN2
 * (per-key-channel gate, independent erase and write gates), chunk size 64,
 * key width up to 128, value width up to 1024, regular or packed
 * variable-length batches.
 *
 * Operation ("ReWY: Faster Backpropagation for Delta-Rule Attention -- From
 * 7 to 3 Matrix Multiplications", paperpeel.com/paper/2611.01940, Sec. 2.2
 * and Table 1; cited below as Sec. / App.). Per batch b and head h, with
 * a key-major state S (128 x 128), for t = 1..T:
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (the output includes the write)
 * with S_0 = h0 and ht = S_T. The gate g is the log decay: one value per
 * token and head (scalar gate) or one per key channel (vector gate). beta is
 * the write weight after its activation; q already carries the query scale.
 * The backward returns the exact gradients of <o, dO> + <ht, dht> with
 * respect to q, k, v, g, beta and h0 (Sec. 3.1: the ReWY backward changes
 * the derivative graph, not the gradients). dg has g's shape; for a scalar
 * gate it is the sum over key channels (App. E.1).
 *
 * Computation: chunkwise (Sec. 2.1, 2.3; the chunk system as the onedev.kr
 * summary of the paper prints it under "How it works") -- per chunk the
 * unit-triangular system M R = Z - E S, A = M^{-1}, W = A E, U = A Z; a state scan across
 * chunks; and a backward whose local producer is the three-product ReWY
 * pullback P = A^T Rbar, P R^T, P S^T (Sec. 3.1-3.2), followed by Gram
 * elimination (scalar gate, Sec. 3.4) or centred matrix intra (vector gate,
 * Sec. 3.3). Dense products run on bf16 MFMA with fp32 accumulation; the
 * triangular inverse, the state and all gate arithmetic are fp32.
 *
 * Layouts (row-major, contiguous, device memory):
 *   q, k, dq, dk        [B, T, H, 128]      dtype
 *   v, o, dO, dv        [B, T, H, 128]      dtype
 *   beta, dbeta         [B, T, H]           dtype
 *   g, dg               [B, T, H] (scalar gate) or [B, T, H, 128] (vector), fp32
 *   h0, ht, dht, dh0    [B, H, 128(key), 128(value)], fp32
 * dtype is GDR_BF16 or GDR_F32 (storage type of the listed tensors; the
 * arithmetic is the same for both).
 *
 * Ownership: every pointer is caller-owned device memory; the library never
 * allocates or frees per call and keeps no state between calls. `saved` and
 * `scratch` are caller-provided workspaces sized by gdr_workspace_size.
 * `saved` must stay untouched between gdr_fwd and the gdr_bwd that uses it.
 * Calls are asynchronous on `stream` (a hipStream_t; NULL = default stream);
 * the library never synchronizes. Concurrent calls must not share `scratch`.
 *
 * Widths: the kernels are built for key and value width 128 (the
 * flashserve/ReWY repository page, "Compatibility": K = V = 128, 64-token
 * chunks). Narrower widths (1 <= DK, DV <= 128; the pages' extended tests
 * use 80/112 and 96/80) run exactly on the same kernels through zero-padded
 * copies in the workspace -- zero key features leave the recurrence
 * unchanged and zero value columns only add zero columns -- at the cost of
 * the padded work and the copies. In the layouts above, 128 then reads DK
 * (q, k, dq, dk, a vector g and dg), DV (v, o, dO, dv) and DK x DV (states).
 * Value widths above 128 (up to 1024) run as 128-wide value blocks: the value
 * columns of the state evolve independently, so each block is its own
 * problem on the same kernels. o, ht, dv and dh0 take the block's columns;
 * the key-side gradients dq, dk, dg and dbeta are the sums of the blocks'
 * contributions, added in block order in fp32 and rounded once per addition
 * to the stored type (no atomics). The key-side work repeats per block, and
 * a full-save `saved` area holds one block's set per block.
 *
 * Errors: arguments are validated before anything is launched; on error
 * nothing is launched and the call returns a negative status. Unsupported
 * shapes (a key width above 128, a value width above 1024, chunk other than
 * 64) return GDR_ERR_UNSUPPORTED
 * -- there is no fallback (that page's "Existing Training Scripts":
 * unsupported configurations fail by default). T may be any length:
 * where that page requires a multiple of 64, a ragged last chunk is handled
 * here, its missing rows acting as identity steps (g = 0, beta = 0, zero
 * q, k, v, dO), which leaves every output, state and gradient of the real
 * tokens exact; workspaces count whole chunks. Vector gate: the centred
 * factors (Sec. 3.3) are formed per 16-token window of the chunk, with
 * boundary pivots between windows, so they span exp(+-range/2) of one
 * window; g must be a log decay (g <= 0) whose per-channel range over each
 * 16-token window is at most 160 (e.g. every |g| <= 10); past that the
 * results are non-finite, not finite and wrong, and gdr_gate_status reports
 * it (the check runs inside the kernels; there is no host synchronization,
 * so the call itself still returns GDR_OK). A launch failure
 * returns GDR_ERR_HIP. gdr_last_error() returns a message for
 * the calling thread's last failure.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_ERR_INVALID = -1,     /* null pointer, negative size, bad enum */
    GDR_ERR_UNSUPPORTED = -2, /* valid but not implemented (see above) */
    GDR_ERR_WORKSPACE = -3,   /* saved/scratch missing or too small */
    GDR_ERR_HIP = -4          /* a HIP launch failed */
} gdr_status;

/* GDR_GATE_NONE: DeltaNet, the recurrence with no decay (g = 0; the pages'
 * Table 1 lists it beside GDN and KDA). g and dg are neither read nor written
 * and may be NULL; the workspace holds a zero log-decay array and a sink for
 * its gradient (8 bytes per token and head), and the scalar-gate kernels run
 * on them. */
/* GDR_GATE_GDN2: GDN2 (the pages' Table 1: per-key-channel log decay with
 * independent erase and write gates); its calls are gdr_fwd_gdn2 and
 * gdr_bwd_gdn2 below, and the beta entry points refuse it. */
typedef enum { GDR_GATE_SCALAR = 0, GDR_GATE_VECTOR = 1, GDR_GATE_NONE = 2, GDR_GATE_GDN2 = 3 } gdr_gate;
typedef enum { GDR_RECOMPUTE = 0, GDR_FULL_SAVE = 1 } gdr_policy;
typedef enum { GDR_BF16 = 0, GDR_F32 = 1 } gdr_dtype;

typedef struct {
    int64_t B, T, H;  /* batch, sequence length, heads */
    int64_t DK, DV;   /* key width 1 .. 128, value width 1 .. 1024 (128: no padding) */
    int64_t C;        /* chunk length: must be 64 */
    int32_t gate;     /* gdr_gate */
    int32_t dtype;    /* gdr_dtype */
} gdr_desc;

/* Workspace sizes in bytes for a descriptor and policy.
 * saved_bytes: what gdr_fwd under GDR_FULL_SAVE writes for gdr_bwd
 *              (0 under GDR_RECOMPUTE).
 * scratch_bytes: transient memory that gdr_fwd / gdr_bwd / gdr_bwd_wy7 need
 *              (the maximum over the three). Any pointer may be NULL. */
int gdr_workspace_size(const gdr_desc* d, int policy, size_t* saved_bytes, size_t* scratch_bytes);

/* Forward. o: output; ht: final state (NULL: not written); h0 NULL: zero.
 * Under GDR_FULL_SAVE, saved receives the chunk quantities the backward
 * reuses (per chunk and head: A^T, Kt, -W, exp(G_n), Hm^T, Qg^T, and the
 * state h and correction R at the chunk; 115,200 bytes at the supported
 * widths); under GDR_RECOMPUTE saved may be NULL. */
int gdr_fwd(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
            const float* g, const void* beta, const float* h0, void* o, float* ht, void* saved,
            void* scratch, size_t scratch_bytes, void* stream);

/* Backward. Under GDR_RECOMPUTE the forward chunk quantities are recomputed
 * into scratch (saved may be NULL); under GDR_FULL_SAVE they are read from
 * saved. dht NULL: zero; dh0 NULL: not written. */
int gdr_bwd(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
            const float* g, const void* beta, const float* h0, const void* dO, const float* dht,
            const void* saved, void* dq, void* dk, void* dv, float* dg, void* dbeta, float* dh0,
            void* scratch, size_t scratch_bytes, void* stream);

/* Same contract and results as gdr_bwd, with the expanded seven-product WY
 * producer (Sec. 2.3: Wbar = -Rbar S^T, Abar = Rbar Z^T + Wbar E^T,
 * Mbar = -A^T Abar A^T, Ebar = A^T Wbar, Zbar = A^T Rbar) in place of ReWY.
 * Ablation only. */
int gdr_bwd_wy7(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                const float* g, const void* beta, const float* h0, const void* dO,
                const float* dht, const void* saved, void* dq, void* dk, void* dv, float* dg,
                void* dbeta, float* dh0, void* scratch, size_t scratch_bytes, void* stream);

/* GDN2 (Sec. 2.2, Table 1: a per-key-channel log decay with an erase gate per
 * key channel and a write gate per value channel, in place of the shared
 * beta; Sec. 3.1 keeps their gradients separate). Per head, for t = 1..T:
 *     St = Diag(exp(g_t)) S_{t-1}
 *     r  = write_t o v_t - St^T (erase_t o k_t)    (prediction from the
 *                                                  erase-gated key, taken from
 *                                                  the write-gated value)
 *     S_t = St + k_t r^T,   o_t = S_t^T q_t
 * which is the vector-gate recurrence when erase_t = write_t = beta_t. The
 * chunk system is the same with E = erase o exp(G) o K and Z = write o V.
 * Layouts: g, dg [B,T,H,DK] fp32; erase, derase [B,T,H,DK] (per key) and
 * write, dwrite [B,T,H,DV] (per value) in bf16, 16-byte aligned; the rest as
 * for gdr_fwd / gdr_bwd, including widths (keys up to 128, values up to 1024)
 * and the packed variable-length form (the _varlen calls, with the offsets
 * and per-sequence states of gdr_fwd_varlen). d->gate must be GDR_GATE_GDN2
 * and d->dtype GDR_BF16 (fp32 storage returns GDR_ERR_UNSUPPORTED); there is
 * no seven-product form. The workspace is gdr_workspace_size(_varlen)'s for
 * the GDN2 descriptor. derase and dwrite are the exact gradients entry by
 * entry; their sums over channels are what a shared beta's gradient would
 * be. */
int gdr_fwd_gdn2(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                 const float* g, const void* erase, const void* write, const float* h0, void* o,
                 float* ht, void* saved, void* scratch, size_t scratch_bytes, void* stream);
int gdr_bwd_gdn2(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                 const float* g, const void* erase, const void* write, const float* h0,
                 const void* dO, const float* dht, const void* saved, void* dq, void* dk, void* dv,
                 float* dg, void* derase, void* dwrite, float* dh0, void* scratch,
                 size_t scratch_bytes, void* stream);
int gdr_fwd_gdn2_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                        const void* q, const void* k, const void* v, const float* g, const void* erase,
                        const void* write, const float* h0, void* o, float* ht, void* saved, void* scratch,
                        size_t scratch_bytes, void* stream);
int gdr_bwd_gdn2_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                        const void* q, const void* k, const void* v, const float* g, const void* erase,
                        const void* write, const float* h0, const void* dO, const float* dht,
                        const void* saved, void* dq, void* dk, void* dv, float* dg, void* derase,
                        void* dwrite, float* dh0, void* scratch, size_t scratch_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): gdr_bwd
 * with no scratch argument. Its scratch is a fixed array of
 * GDR_NOALLOC_SCRATCH_MAX bytes inside the library, one per device, held
 * from the library's first use on that device until the process ends; the
 * call itself allocates nothing. Same arguments (minus scratch), results and
 * errors as gdr_bwd for a regular batch; the stream must belong to the
 * current device (else GDR_ERR_INVALID). A problem whose gdr_bwd scratch
 * (gdr_workspace_size) exceeds the array returns GDR_ERR_UNSUPPORTED before
 * anything is launched: about 310 (chunk, head) pairs under GDR_RECOMPUTE,
 * e.g. (B, T, H) = (1, 2048, 9), about 630 under GDR_FULL_SAVE. Every call on
 * one device shares that device's array and leaves its contents behind (the
 * kernels write every part they read before reading it), so calls that
 * overlap in time on one device -- on two streams, or from two threads --
 * race on it and must not be issued. */
#define GDR_NOALLOC_SCRATCH_MAX ((size_t)64 << 20)
int gdr_bwd_noalloc(const gdr_desc* d, int policy, const void* q, const void* k, const void* v,
                    const float* g, const void* beta, const float* h0, const void* dO,
                    const float* dht, const void* saved, void* dq, void* dk, void* dv, float* dg,
                    void* dbeta, float* dh0, void* stream);

/* Packed variable-length batches (several sequences in one row of tokens,
 * the cu_seqlens convention of flash-linear-attention, which the pages'
 * reference implementation builds on). d->B must be 1; the row of d->T
 * tokens holds n_seq sequences, sequence i spanning tokens
 * [cu_seqlens[i], cu_seqlens[i+1]). cu_seqlens is a DEVICE array of n_seq + 1
 * int64 offsets, 8-byte aligned, expected nondecreasing from 0 (the library
 * reads it only on the device, clamps it to [0, T] and makes it
 * nondecreasing, so malformed offsets cannot make it read or write outside
 * the tensors; tokens outside every sequence are left untouched). Each
 * sequence is chunked on its own (its last chunk may be ragged) and starts
 * from its own state: h0, ht, dht, dh0 are [n_seq, H, 128, 128] fp32.
 * Empty sequences pass their state through. Everything else (tensors,
 * dtypes, policies, errors) is as for gdr_fwd / gdr_bwd. The workspace
 * holds ceil(T / 64) + n_seq chunk slots per head plus small sequence
 * tables; a full-save `saved` area is tied to the cu_seqlens it was written
 * with. */
int gdr_workspace_size_varlen(const gdr_desc* d, int64_t n_seq, int policy, size_t* saved_bytes,
                              size_t* scratch_bytes);
int gdr_fwd_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                   const void* q, const void* k, const void* v, const float* g, const void* beta,
                   const float* h0, void* o, float* ht, void* saved, void* scratch,
                   size_t scratch_bytes, void* stream);
int gdr_bwd_varlen(const gdr_desc* d, int policy, const int64_t* cu_seqlens, int64_t n_seq,
                   const void* q, const void* k, const void* v, const float* g, const void* beta,
                   const float* h0, const void* dO, const float* dht, const void* saved, void* dq,
                   void* dk, void* dv, float* dg, void* dbeta, float* dh0, void* scratch,
                   size_t scratch_bytes, void* stream);

/* Per-stage timing for benchmarks. gdr_profile_begin creates 2*max_launches
 * HIP events (the only allocation the library makes, and only here) and
 * turns timing on: every kernel that gdr_fwd / gdr_bwd / gdr_bwd_wy7 then
 * launch is bracketed by events recorded on the call's stream. Stages are
 * "prep", "scan_fwd", "xy", "scan_bwd", "scan_pair" (both scans of the
 * recompute backward in one launch), "bwd_local", "bwd_local_wy7", "pad" (the
 * copies of widths below 128), "a_from_at" (the full-save seven-product
 * backward's A from the saved A^T).
 * gdr_profile_end turns timing off, waits for the recorded events (a host
 * synchronization), and writes up to `cap` per-stage totals; *n_out receives
 * the number of stages seen. Launches beyond max_launches run untimed and
 * gdr_profile_end then returns GDR_ERR_WORKSPACE (totals still written).
 * Not meant to be combined with stream capture. */
typedef struct {
    char name[32];
    int64_t launches;
    double total_ms;
} gdr_stage_time;
int gdr_profile_begin(int max_launches);
int gdr_profile_end(gdr_stage_time* out, int cap, int* n_out);

/* Gate-range status. The chunk preparation of every gdr_fwd*, gdr_bwd* under
 * GDR_RECOMPUTE and gdr_bwd_noalloc records, per chunk and head, whether the
 * log decays it read leave the contract above (ReWY paper Sec. 3.3
 * "Centered factors": the implementation checks gate ranges; the repository
 * page, "Compatibility": unsupported configurations fail). The words sit in
 * `scratch` and cost no extra pass or synchronization. gdr_gate_status ORs
 * those of the last such call made with this descriptor and scratch into
 * *status (a DEVICE int32, written asynchronously on `stream`):
 *   GDR_GATE_POSITIVE   a log decay above 0
 *   GDR_GATE_RANGE      vector gate (and GDN2): a 16-token window whose
 *                       per-channel range exceeds 160
 *   GDR_GATE_NONFINITE  a log decay that is NaN or infinite
 * and 0 when every decay was within it. n_seq: the sequence count of a
 * packed batch (the offsets the call ran with), or -1 for a regular batch.
 * A gdr_bwd under GDR_FULL_SAVE reads no gates (its forward checked them).
 * Results computed past GDR_GATE_RANGE or GDR_GATE_NONFINITE are not
 * meaningful; a positive decay within range is computed as given. */
enum { GDR_GATE_POSITIVE = 1, GDR_GATE_RANGE = 2, GDR_GATE_NONFINITE = 4 };
int gdr_gate_status(const gdr_desc* d, int64_t n_seq, const void* scratch, size_t scratch_bytes,
                    int32_t* status, void* stream);

/* Launch form of the scalar-gate three-product local backward, for
 * like-for-like timing of the ablation (process-wide; set it between calls,
 * not during one). GDR_LOCAL_PERSISTENT (the default): one workgroup per
 * compute unit walks its share of the (chunk, head) items and streams the
 * next item's per-chunk states into LDS meanwhile. GDR_LOCAL_PER_CHUNK: one
 * workgroup per (chunk, head), the form the vector-gate and seven-product
 * local kernels always use. Both compute the same arithmetic; the two
 * instantiations may round the fp32 gate and beta reductions differently
 * in the last bits.
 * Returns the previous form, or GDR_ERR_INVALID for an unknown one. */
typedef enum { GDR_LOCAL_PERSISTENT = 0, GDR_LOCAL_PER_CHUNK = 1 } gdr_local_form;
int gdr_set_local_form(int form);

/* Form of the state walks (process-wide; set it between calls, not during
 * one). The walks are serial over a sequence's chunks (Sec. 2.1). A walk
 * launch over few (sequence, head) pairs leaves most compute units idle;
 * GDR_WALK_AUTO (the default) then cuts each walk of a regular batch into
 * segments: the map from a segment's entry state to its exit state (its
 * homogeneous part, keys x keys, and its exit state from zero) is formed for
 * all segments at once, the segments' entry states are chained through those
 * maps in fp32, and every segment then walks from its own entry state. This
 * applies when the one-level launch would fill at most a quarter of 256
 * compute units and the walk is long enough for 3 or more segments of at
 * least 8 chunks (for example (1, 8192, 4)). GDR_WALK_ONE_LEVEL walks every
 * sequence start to end. Both give the same results up to rounding; the
 * workspace is sized for the automatic form either way.
 * Returns the previous form, or GDR_ERR_INVALID for an unknown one. */
typedef enum { GDR_WALK_AUTO = 0, GDR_WALK_ONE_LEVEL = 1 } gdr_walk_levels;
int gdr_set_walk_levels(int levels);

const char* gdr_status_string(int status);
const char* gdr_last_error(void);
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
