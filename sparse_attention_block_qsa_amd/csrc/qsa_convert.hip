// qsa_convert.hip -- fp32 -> fp16 conversion of the query activations, the
// "fp16 conversion" stage of the QSA select phase (Strata pull request #228,
// part 1, paragraph after the bench table).  HBM-bound streaming kernel:
// 32 bytes in, 16 bytes out per lane per iteration, grid-stride.
#include "qsa_internal.h"

namespace qsa {
namespace {

// Round to nearest even.  v_cvt_f16_f32 rounds by the MODE register, which
// is round-to-nearest-even for compute kernels, keeps fp16 subnormals and
// overflows to infinity.  NaN is rewritten explicitly so its bits are
// defined: quiet, with the sign and the top 10 fraction bits of the input.
__device__ __forceinline__ uint32_t f16_rne(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    uint32_t h = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    if ((u & 0x7fffffffu) > 0x7f800000u)
        h = ((u >> 16) & 0x8000u) | 0x7e00u | ((u >> 13) & 0x3ffu);
    return h;
}

__global__ __launch_bounds__(256) void convert_v8_kernel(const float4 *__restrict__ src,
                                                          uint4 *__restrict__ dst, int64_t n8) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n8; i += stride) {
        const float4 a = src[2 * i];
        const float4 b = src[2 * i + 1];
        uint4 o;
        o.x = f16_rne(a.x) | (f16_rne(a.y) << 16);
        o.y = f16_rne(a.z) | (f16_rne(a.w) << 16);
        o.z = f16_rne(b.x) | (f16_rne(b.y) << 16);
        o.w = f16_rne(b.z) | (f16_rne(b.w) << 16);
        dst[i] = o;
    }
}

__global__ __launch_bounds__(256) void convert_scalar_kernel(const float *__restrict__ src,
                                                              uint16_t *__restrict__ dst,
                                                              int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
        dst[i] = static_cast<uint16_t>(f16_rne(src[i]));
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

}  // namespace qsa
