// Key / value widths below 128: zero-padded copies. Zero key features leave
// the recurrence exact -- their state rows receive no writes and their query
// features read nothing -- and zero value columns only add state and output
// columns of zeros, so a problem with d_k, d_v <= 128 runs on the 128-wide
// kernels through these copies (gdr_api.hip). Bit copies: the element type
// only sets the width (2 bytes for bf16, 4 for fp32), and zero bits are 0.
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

// rows of width w -> rows of width 128, zeros past w
template <typename E>
__global__ void pad_rows_kernel(E* dst, const E* src, int64_t rows, int w)
{
    const int64_t n = rows * W;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / W;
        const int f = (int)(i - r * W);
        dst[i] = f < w ? src[r * w + f] : E(0);
    }
}

// rows of width 128 -> rows of width w (the first w entries)
template <typename E>
__global__ void unpad_rows_kernel(E* dst, const E* src, int64_t rows, int w)
{
    const int64_t n = rows * w;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / w;
        const int f = (int)(i - r * w);
        dst[i] = src[r * W + f];
    }
}

// states [n][dk][dv] -> [n][128][128], zeros elsewhere
__global__ void pad_state_kernel(float* dst, const float* src, int64_t n, int dk, int dv)
{
    const int64_t tot = n * W * W;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / (W * W);
        const int rem = (int)(i - s * (W * W)), a = rem / W, b = rem - a * W;
        dst[i] = (a < dk && b < dv) ? src[(s * dk + a) * dv + b] : 0.f;
    }
}

// states [n][128][128] -> [n][dk][dv]
__global__ void unpad_state_kernel(float* dst, const float* src, int64_t n, int dk, int dv)
{
    const int64_t tot = n * dk * dv;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < tot; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t s = i / ((int64_t)dk * dv);
        const int rem = (int)(i - s * dk * dv), a = rem / dv, b = rem - a * dv;
        dst[i] = src[(s * W + a) * W + b];
    }
}

}  // namespace

hipError_t launch_pad_rows(void* dst, const void* src, int64_t rows, int w, int esz, hipStream_t st)
{
    if (esz == 2)
        pad_rows_kernel<uint16_t><<<grid_for(rows * W), 256, 0, st>>>((uint16_t*)dst, (const uint16_t*)src, rows, w);
    else
        pad_rows_kernel<uint32_t><<<grid_for(rows * W), 256, 0, st>>>((uint32_t*)dst, (const uint32_t*)src, rows, w);
    return hipGetLastError();
}

hipError_t launch_unpad_rows(void* dst, const void* src, int64_t rows, int w, int esz, hipStream_t st)
{
    if (esz == 2)
        unpad_rows_kernel<uint16_t><<<grid_for(rows * w), 256, 0, st>>>((uint16_t*)dst, (const uint16_t*)src, rows, w);
    else
        unpad_rows_kernel<uint32_t><<<grid_for(rows * w), 256, 0, st>>>((uint32_t*)dst, (const uint32_t*)src, rows, w);
    return hipGetLastError();
}

hipError_t launch_pad_state(float* dst, const float* src, int64_t n, int dk, int dv, hipStream_t st)
{
    pad_state_kernel<<<grid_for(n * W * W), 256, 0, st>>>(dst, src, n, dk, dv);
    return hipGetLastError();
}

hipError_t launch_unpad_state(float* dst, const float* src, int64_t n, int dk, int dv, hipStream_t st)
{
    unpad_state_kernel<<<grid_for(n * dk * dv), 256, 0, st>>>(dst, src, n, dk, dv);
    return hipGetLastError();
}

}  // namespace gdr
