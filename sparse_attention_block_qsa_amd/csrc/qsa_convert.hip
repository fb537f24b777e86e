// qsa_convert.hip -- fp32 -> fp16 conversion of the query activations, the
// "fp16 conversion" stage of the QSA select phase (Strata pull request #228,
// part 1, paragraph after the bench table).  HBM-bound streaming kernels:
// 32 bytes in, 16 bytes out per lane per iteration, grid-stride; the phase
// converts exactly the token rows of a strided query tensor.
#include "qsa_internal.h"

namespace qsa {
namespace {

__global__ __launch_bounds__(256) void convert_v8_kernel(const float4 *__restrict__ src,
                                                          uint4 *__restrict__ dst, int64_t n8) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8; i += stride) {
        const float4 a = src[2 * i];
        const float4 b = src[2 * i + 1];
        dst[i] = f16x8(a, b);   // the scorers' on-load conversion
    }
}

__global__ __launch_bounds__(256) void convert_scalar_kernel(const float *__restrict__ src,
                                                              uint16_t *__restrict__ dst,
                                                              int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
        dst[i] = static_cast<uint16_t>(f16_rne(src[i]));
}

// Token rows of a strided query tensor: element e of row r at r * stride + e.
__global__ __launch_bounds__(256) void convert_rows_kernel(const float *__restrict__ src,
                                                            uint16_t *__restrict__ dst,
                                                            int64_t n, int64_t row_len,
                                                            int64_t stride) {
    const int64_t step = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += step) {
        const int64_t r = i / row_len;
        const int64_t off = r * stride + (i - r * row_len);
        dst[off] = static_cast<uint16_t>(f16_rne(src[off]));
    }
}

unsigned grid_for(int64_t items) {
    int64_t blocks = (items + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    return static_cast<unsigned>(blocks < 1 ? 1 : blocks);
}

}  // namespace

hipError_t launch_convert(const float *src, uint16_t *dst, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t done = 0;
    const bool aligned = (reinterpret_cast<uintptr_t>(src) % 16 == 0) &&
                         (reinterpret_cast<uintptr_t>(dst) % 16 == 0);
    if (aligned && n >= 8) {
        const float4 *s4 = reinterpret_cast<const float4 *>(src);
        uint4 *d4 = reinterpret_cast<uint4 *>(dst);
        int64_t n8 = n / 8;
        void *args[] = {&s4, &d4, &n8};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&convert_v8_kernel),
                                       dim3(grid_for(n8)), dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
        done = n8 * 8;
    }
    if (done < n) {
        const float *st = src + done;
        uint16_t *dt = dst + done;
        int64_t rem = n - done;
        void *args[] = {&st, &dt, &rem};
        return hipLaunchKernel(reinterpret_cast<const void *>(&convert_scalar_kernel),
                               dim3(grid_for(rem)), dim3(256), args, 0, s);
    }
    return hipSuccess;
}

hipError_t launch_convert_rows(const float *src, uint16_t *dst, int64_t rows, int64_t row_len,
                               int64_t stride, hipStream_t s) {
    if (rows <= 0 || row_len <= 0) return hipSuccess;
    if (stride == row_len) return launch_convert(src, dst, rows * row_len, s);
    int64_t n = rows * row_len;
    void *args[] = {&src, &dst, &n, &row_len, &stride};
    return hipLaunchKernel(reinterpret_cast<const void *>(&convert_rows_kernel),
                           dim3(grid_for(n)), dim3(256), args, 0, s);
}

}  // namespace qsa
