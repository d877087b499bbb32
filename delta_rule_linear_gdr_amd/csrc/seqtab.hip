// Packed variable-length batches (several sequences in one row of T tokens,
// FLA's cu_seqlens convention): the sequence and chunk-slot tables every
// other kernel reads (kernels.h, Shape::cu / stab / ctab / order). One
// workgroup; N + 1 offsets are processed in tiles of 1024 with a running
// carry.
//
// `order` lists the sequences longest first, so that the scans, whose
// workgroups each walk one sequence's chunks serially, start the longest
// walks first (longest-processing-time-first list scheduling). Lengths are
// ranked by class -- the chunk count itself below 4, else its octave and the
// two bits after the leading one -- which keeps the ranking a single
// histogram pass; ties within a class are placed in any order (only the
// schedule depends on it, never a result).
//
// The caller's offsets are sanitized first (clamped to [0, T], cu[0] = 0,
// made nondecreasing), so no table entry can send a kernel outside the
// tensors or the chunk slots whatever the offsets hold: the slots of all
// sequences number at most ceil(T / 64) + N.
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int NTH = 1024;
constexpr int NCLASS = 128;

// Length class of a chunk count n < 2^30; nondecreasing in n, below NCLASS.
__device__ __forceinline__ int len_class(int n)
{
    if (n < 4) return n;
    const int e = 31 - __clz(n);
    return 4 * (e - 1) + ((n >> (e - 2)) & 3);
}

// Inclusive block scan of x over the 1024 threads with `op`; every thread
// also receives the tile total in *tot.
template <typename Op>
__device__ int64_t block_scan(int64_t x, int64_t* buf, int64_t* tot, Op op)
{
    const int tid = threadIdx.x;
    __syncthreads();  // buf may still be read from the previous call
    buf[tid] = x;
    __syncthreads();
    for (int off = 1; off < NTH; off <<= 1) {
        const int64_t y = tid >= off ? buf[tid - off] : 0;
        __syncthreads();
        if (tid >= off) buf[tid] = op(buf[tid], y);
        __syncthreads();
    }
    *tot = buf[NTH - 1];
    return buf[tid];
}

__global__ __launch_bounds__(NTH) void seq_tables_kernel(Shape s, const int64_t* cu_in, int64_t* cu,
                                                         int2* stab, int2* ctab, int* order)
{
    __shared__ int64_t buf[NTH];
    __shared__ int cls_next[NCLASS];
    const int tid = threadIdx.x;
    const int64_t N = s.NS, T = s.T;
    auto mx = [](int64_t a, int64_t b) { return a > b ? a : b; };
    auto add = [](int64_t a, int64_t b) { return a + b; };

    // 1. cu[i] = max over j <= i of clamp(cu_in[j], 0, T), with cu[0] = 0
    int64_t carry = 0;
    for (int64_t base = 0; base <= N; base += NTH) {
        const int64_t i = base + tid;
        int64_t x = 0;
        if (i <= N && i > 0) {
            x = cu_in[i];
            x = x < 0 ? 0 : x > T ? T : x;
        }
        int64_t tot;
        const int64_t m = mx(block_scan(x, buf, &tot, mx), carry);
        if (i <= N) cu[i] = m;
        carry = mx(carry, tot);
    }
    __syncthreads();  // cu complete (workgroup-scope fence included)

    // 2. per sequence: chunk count and first slot (exclusive sum)
    carry = 0;
    for (int64_t base = 0; base < N; base += NTH) {
        const int64_t i = base + tid;
        int64_t nc = 0;
        if (i < N) nc = (cu[i + 1] - cu[i] + CH - 1) / CH;
        int64_t tot;
        const int64_t incl = block_scan(nc, buf, &tot, add);
        if (i < N) stab[i] = make_int2((int)(carry + incl - nc), (int)nc);
        carry += tot;
    }

    // 3. chunk slots: unused (no rows) by default, then each sequence claims
    //    its own: {token of the chunk's row 0, rows} (tokens < 2^31, checked
    //    by the caller)
    for (int64_t j = tid; j < s.NC; j += NTH) ctab[j] = make_int2(0, 0);
    if (tid < NCLASS) cls_next[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < N; i += NTH) {
        const int2 e = stab[i];
        const int64_t tok = cu[i], len = cu[i + 1] - tok;
        for (int c = 0; c < e.y; ++c) {
            const int64_t rows = len - (int64_t)c * CH;
            ctab[e.x + c] = make_int2((int)(tok + (int64_t)c * CH), rows < CH ? (int)rows : CH);
        }
        atomicAdd(&cls_next[len_class(e.y)], 1);
    }
    __syncthreads();

    // 4. order: class counts -> first position of each class, longest first
    if (tid == 0) {
        int pos = 0;
        for (int k = NCLASS - 1; k >= 0; --k) {
            const int n = cls_next[k];
            cls_next[k] = pos;
            pos += n;
        }
    }
    __syncthreads();
    for (int64_t i = tid; i < N; i += NTH) order[atomicAdd(&cls_next[len_class(stab[i].y)], 1)] = (int)i;
}

}  // namespace

hipError_t launch_seq_tables(const Shape& s, const int64_t* cu_in, int64_t* cu, int2* stab, int2* ctab,
                             int* order, hipStream_t st)
{
    seq_tables_kernel<<<1, NTH, 0, st>>>(s, cu_in, cu, stab, ctab, order);
    return hipGetLastError();
}

}  // namespace gdr
