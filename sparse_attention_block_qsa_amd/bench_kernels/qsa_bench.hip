// qsa_bench.hip -- measurement kernels for the benchmark (libqsa_bench.so),
// not part of the select phase: they give the benchmark measured ceilings to
// set the phase's kernels against, beside the published peaks.
//
//  * qsa_bench_mfma_f16 / qsa_bench_mfma_f16_16x16x32: a loop of
//    v_mfma_f32_32x32x16_f16 or v_mfma_f32_16x16x32_f16 (the scorers'
//    instructions) on register-resident operands, no memory traffic: the
//    sustained dense fp16 matrix rate of the chip.  The operands are read
//    once from a caller buffer, so random fp16 data and zeros can be
//    compared (the chip's clock depends on how much the datapath toggles,
//    and under the power limit the two shapes sustain different rates).
//  * qsa_bench_read: a streaming read of a buffer, 16 bytes per lane per
//    load: the achievable HBM read bandwidth for a buffer larger than the
//    last-level cache.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Each wave holds four A and four B fragments (lane-distinct) and cycles
// through all sixteen (A, B) pairs into four independent accumulators, so
// no MFMA waits for the previous one's result.
// held = 1: every MFMA of a wave takes the same A and B fragment (the
// datapath toggles least); held = 0: four A and four B fragments in turn.
__global__ __launch_bounds__(256) void mfma_f16_kernel(const uint4 *ops, int64_t n_ops, float *out,
                                                       int iters, int held) {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    half8 a[4], b[4];
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t ja = held ? 0 : j;
        a[j] = __builtin_bit_cast(half8, ops[(tid * 8 + ja) % n_ops]);
        b[j] = __builtin_bit_cast(half8, ops[(tid * 8 + 4 + ja) % n_ops]);
    }
    floatx16 c[4] = {};
    for (int it = 0; it < iters; ++it) {
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            #pragma unroll
            for (int j = 0; j < 4; ++j)
                c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[(i + j) & 3], c[j], 0, 0, 0);
        }
    }
    float s = 0.0f;
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        #pragma unroll
        for (int r = 0; r < 16; ++r) s += c[j][r];
    }
    out[tid] = s;   // keeps the loop alive
}

// The same loop on v_mfma_f32_16x16x32_f16 (half the FLOP per instruction):
// eight accumulators, each taken every eighth MFMA.
__global__ __launch_bounds__(256) void mfma_f16_16x16x32_kernel(const uint4 *ops, int64_t n_ops,
                                                                float *out, int iters, int held) {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    half8 a[4], b[4];
    #pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t ja = held ? 0 : j;
        a[j] = __builtin_bit_cast(half8, ops[(tid * 8 + ja) % n_ops]);
        b[j] = __builtin_bit_cast(half8, ops[(tid * 8 + 4 + ja) % n_ops]);
    }
    floatx4 c[8] = {};
    for (int it = 0; it < iters; ++it) {
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            #pragma unroll
            for (int j = 0; j < 4; ++j)
                c[(i & 1) * 4 + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[(i + j) & 3],
                                                                            c[(i & 1) * 4 + j], 0, 0, 0);
        }
    }
    float s = 0.0f;
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        #pragma unroll
        for (int r = 0; r < 4; ++r) s += c[j][r];
    }
    out[tid] = s;   // keeps the loop alive
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void read_kernel(const u32x4 *src, int64_t n, uint32_t *out) {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    uint32_t x = 0;
    for (int64_t i = tid; i < n; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[tid] = x;
}

// Does nothing: its launches measure the fixed cost of a launch, the floor
// under every latency-bound kernel.
__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// MFMAs issued per thread-loop iteration by each wave: 16.
int qsa_bench_mfma_per_iter(void) { return 16; }

// grid workgroups of 256 threads; ops: n_ops 16-byte fp16 fragments;
// out: grid*256 floats; held: see mfma_f16_kernel.  Returns a HIP error
// code (0 = launched).
int qsa_bench_mfma_f16(const void *ops, int64_t n_ops, float *out, int grid, int iters,
                       int held, void *stream) {
    if (!ops || !out || n_ops < 1 || grid < 1 || iters < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_f16_kernel, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(ops), n_ops,
                       out, iters, held);
    return hipGetLastError();
}

// The same for the 16x16x32 loop (16 MFMAs of 16x16x32 per iteration).
int qsa_bench_mfma_f16_16x16x32(const void *ops, int64_t n_ops, float *out, int grid, int iters,
                                int held, void *stream) {
    if (!ops || !out || n_ops < 1 || grid < 1 || iters < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_f16_16x16x32_kernel, dim3(grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4 *>(ops), n_ops,
                       out, iters, held);
    return hipGetLastError();
}

// src: n 16-byte units; out: grid*256 uint32.
int qsa_bench_read(const void *src, int64_t n, uint32_t *out, int grid, void *stream) {
    if (!src || !out || n < 1 || grid < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), n, out);
    return hipGetLastError();
}

// grid workgroups of block threads of a kernel with no work.
int qsa_bench_empty(int grid, int block, void *stream) {
    if (grid < 1 || block < 1 || block > 1024) return hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(block), 0, static_cast<hipStream_t>(stream));
    return hipGetLastError();
}

}  // extern "C"
