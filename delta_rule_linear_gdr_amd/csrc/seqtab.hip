// Packed variable-length batches (several sequences in one row of T tokens,
// FLA's cu_seqlens convention): the sequence and chunk-slot tables every
// other kernel reads (kernels.h, Shape::cu / stab / ctab). One workgroup;
// N + 1 offsets are processed in tiles of 1024 with a running carry.
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
                                                         int2* stab, int2* ctab)
{
    __shared__ int64_t buf[NTH];
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

    // 3. chunk slots: unused by default, then each sequence claims its own
    for (int64_t j = tid; j < s.NC; j += NTH) ctab[j] = make_int2(-1, 0);
    __syncthreads();
    for (int64_t i = tid; i < N; i += NTH) {
        const int2 e = stab[i];
        for (int c = 0; c < e.y; ++c) ctab[e.x + c] = make_int2((int)i, c);
    }
}

}  // namespace

hipError_t launch_seq_tables(const Shape& s, const int64_t* cu_in, int64_t* cu, int2* stab, int2* ctab,
                             hipStream_t st)
{
    seq_tables_kernel<<<1, NTH, 0, st>>>(s, cu_in, cu, stab, ctab);
    return hipGetLastError();
}

}  // namespace gdr
