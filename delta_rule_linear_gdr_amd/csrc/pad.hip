// Key / value widths other than 128: zero-padded copies. Zero key features
// leave the recurrence exact -- their state rows receive no writes and their
// query features read nothing -- and zero value columns only add state and
// output columns of zeros, so a problem with d_k, d_v <= 128 runs on the
// 128-wide kernels through these copies (gdr_api.hip). Value columns of the
// state evolve independently, so a value width above 128 runs as 128-wide
// value blocks: the copies then take a block (a column offset into wider
// rows), and the key-side gradients of the blocks are summed (ADD). Plain
// copies are bit copies: the element type only sets the width (2 bytes for
// bf16, 4 for fp32), and zero bits are 0. For a packed batch the copies out
// stop at the end of the last sequence (`end`, the sanitized offsets' last
// entry, read on the device; rows are token-major with `per` rows a token):
// tokens past it are outside every sequence and keep their contents.
#include "common.h"
#include "kernels.h"

namespace gdr {

namespace {

constexpr int W = DKD;  // padded width (keys and values alike)

unsigned grid_for(int64_t n)
{
    int64_t b = (n + 255) / 256;
    return (unsigned)(b < 1 ? 1 : b > 8192 ? 8192 : b);
}

// rows of width w, taken from column col0 of rows of src_ld entries ->
// rows of width 128, zeros past w
template <typename E>
__global__ void pad_rows_kernel(E* dst, const E* src, int64_t rows, int w, int src_ld, int col0)
{
    const int64_t n = rows * W;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / W;
        const int f = (int)(i - r * W);
        dst[i] = f < w ? src[r * src_ld + col0 + f] : E(0);
    }
}

// rows of width 128 -> the first w entries, to column col0 of rows of dst_ld
// entries (a copy, or with ADD the sum dst + src rounded once to the type)
template <typename E, bool ADD>
__global__ void unpad_rows_kernel(E* dst, const E* src, int64_t rows, int w, int dst_ld, int col0,
                                  const int64_t* end, int per)
{
    if (end) rows = min(rows, *end * per);
    const int64_t n = rows * w;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / w;
        const int f = (int)(i - r * w);
        E* d = dst + r * dst_ld + col0 + f;
        if (ADD) *d = (E)((float)*d + (float)src[r * W + f]);
        else *d = src[r * W + f];
    }
}

// states [n][dk][src_dv] (value columns col0 .. col0 + dv) -> [n][128][128],
// zeros elsewhere
__global__ void pad_state_kernel(float* dst, const float* src, int64_t n, int dk, int dv, int src_dv, int col0)
{
    const int64_t tot = n * W * W;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / (W * W);
        const int rem = (int)(i - s * (W * W)), a = rem / W, b = rem - a * W;
        dst[i] = (a < dk && b < dv) ? src[(s * dk + a) * src_dv + col0 + b] : 0.f;
    }
}

// states [n][128][128] -> value columns col0 .. col0 + dv of [n][dk][dst_dv]
__global__ void unpad_state_kernel(float* dst, const float* src, int64_t n, int dk, int dv, int dst_dv, int col0)
{
    const int64_t tot = n * dk * dv;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / ((int64_t)dk * dv);
        const int rem = (int)(i - s * dk * dv), a = rem / dv, b = rem - a * dv;
        dst[(s * dk + a) * dst_dv + col0 + b] = src[(s * W + a) * W + b];
    }
}

// dst[i] += src[i], i < n, rounded once to the type
template <typename E>
__global__ void add_entries_kernel(E* dst, const E* src, int64_t n, const int64_t* end, int per)
{
    if (end) n = min(n, *end * per);
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = (E)((float)dst[i] + (float)src[i]);
}

}  // namespace

hipError_t launch_add_entries(void* dst, const void* src, int64_t n, int esz, hipStream_t st, const int64_t* end,
                              int per)
{
    if (esz == 2) add_entries_kernel<bf16><<<grid_for(n), 256, 0, st>>>((bf16*)dst, (const bf16*)src, n, end, per);
    else add_entries_kernel<float><<<grid_for(n), 256, 0, st>>>((float*)dst, (const float*)src, n, end, per);
    return hipGetLastError();
}

hipError_t launch_pad_rows(void* dst, const void* src, int64_t rows, int w, int esz, hipStream_t st,
                           int src_ld, int col0)
{
    if (src_ld <= 0) src_ld = w;
    if (esz == 2)
        pad_rows_kernel<uint16_t><<<grid_for(rows * W), 256, 0, st>>>((uint16_t*)dst, (const uint16_t*)src, rows, w,
                                                                      src_ld, col0);
    else
        pad_rows_kernel<uint32_t><<<grid_for(rows * W), 256, 0, st>>>((uint32_t*)dst, (const uint32_t*)src, rows, w,
                                                                      src_ld, col0);
    return hipGetLastError();
}

hipError_t launch_unpad_rows(void* dst, const void* src, int64_t rows, int w, int esz, hipStream_t st,
                             int dst_ld, int col0, bool add, const int64_t* end, int per)
{
    if (dst_ld <= 0) dst_ld = w;
    const unsigned gr = grid_for(rows * w);
    if (add) {
        // sums need the element type: bf16 (2 bytes) or fp32 (4)
        if (esz == 2)
            unpad_rows_kernel<bf16, true><<<gr, 256, 0, st>>>((bf16*)dst, (const bf16*)src, rows, w, dst_ld, col0,
                                                              end, per);
        else
            unpad_rows_kernel<float, true><<<gr, 256, 0, st>>>((float*)dst, (const float*)src, rows, w, dst_ld, col0,
                                                               end, per);
    } else if (esz == 2) {
        unpad_rows_kernel<uint16_t, false><<<gr, 256, 0, st>>>((uint16_t*)dst, (const uint16_t*)src, rows, w, dst_ld,
                                                              col0, end, per);
    } else {
        unpad_rows_kernel<uint32_t, false><<<gr, 256, 0, st>>>((uint32_t*)dst, (const uint32_t*)src, rows, w, dst_ld,
                                                              col0, end, per);
    }
    return hipGetLastError();
}

hipError_t launch_pad_state(float* dst, const float* src, int64_t n, int dk, int dv, hipStream_t st, int src_dv,
                            int col0)
{
    if (src_dv <= 0) src_dv = dv;
    pad_state_kernel<<<grid_for(n * W * W), 256, 0, st>>>(dst, src, n, dk, dv, src_dv, col0);
    return hipGetLastError();
}

hipError_t launch_unpad_state(float* dst, const float* src, int64_t n, int dk, int dv, hipStream_t st, int dst_dv,
                              int col0)
{
    if (dst_dv <= 0) dst_dv = dv;
    unpad_state_kernel<<<grid_for(n * dk * dv), 256, 0, st>>>(dst, src, n, dk, dv, dst_dv, col0);
    return hipGetLastError();
}

}  // namespace gdr
