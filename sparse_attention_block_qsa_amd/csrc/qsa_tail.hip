// qsa_tail.hip -- the separate scorer of the partial last KV block.
//
// The pages score the block holding the last n_kv mod bs tokens with its own
// shared kernel whose result is bitwise reproducible (Strata pull request
// #228, part 1, the paragraph naming the tail kernel; pull request #856,
// "What").  Here its order is fixed by construction, per (query, KV head):
//   acc_h = +0;  for i ascending: acc_h = fma(k[i], q_h[i], acc_h)   (fp32)
//   r_h   = acc_h > 0 ? acc_h : +0
//   s     = +0;  for h ascending: s = s + r_h
// One lane runs one (query, head) chain.  The queries of a workgroup are
// read once, fully coalesced, into LDS (one padded row of D fp16 per chain),
// then every lane walks its own row; a second LDS pass sums the heads of each
// query in order.  HBM-bound: it reads 2*H*D bytes per query row.
#include "qsa_internal.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

struct TailArgs {
    const uint16_t *q16;
    int64_t qts;
    const uint16_t *kblk;
    int64_t khs;
    float *scores;
    int64_t ld_s;
    int32_t G, nq, H;
    int64_t b_tail;
    int32_t rows_per_wg;
};

template <int D>
__global__ __launch_bounds__(256) void tail_kernel(TailArgs a) {
    constexpr int C8 = D / 8;          // uint4 per chain row
    constexpr int PITCH = C8 + 1;      // padded: conflict-free ds_read_b128
    __shared__ uint4 qs[256 * PITCH];
    __shared__ float red[256];

    const int g = blockIdx.y;
    const int R = a.rows_per_wg;
    const int t0 = blockIdx.x * R;
    const int HC8 = a.H * C8;          // uint4 per query row

    // coalesced load of R query rows (H*D fp16 each, contiguous per row)
    const int total = R * HC8;
    for (int u = threadIdx.x; u < total; u += 256) {
        const int rho = u / HC8, wv = u % HC8;
        const int t = t0 + rho;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (t < a.nq)
            v = *reinterpret_cast<const uint4 *>(a.q16 + static_cast<int64_t>(t) * a.qts +
                                                 static_cast<int64_t>(g) * a.H * D + 8 * wv);
        const int chain = rho * a.H + wv / C8;
        qs[chain * PITCH + wv % C8] = v;
    }
    __syncthreads();

    const int c = threadIdx.x;
    const uint16_t *kb = a.kblk + static_cast<int64_t>(g) * a.khs + a.b_tail * D;
    if (c < R * a.H) {
        float acc = 0.0f;
        #pragma unroll
        for (int j = 0; j < C8; ++j) {
            const uint4 qv = qs[c * PITCH + j];
            const uint4 kv = *reinterpret_cast<const uint4 *>(kb + 8 * j);
            const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
            const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(qw[e] & 0xffffu)));
                const float q1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(qw[e] >> 16)));
                const float k0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kw[e] & 0xffffu)));
                const float k1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kw[e] >> 16)));
                acc = __builtin_fmaf(k0, q0, acc);
                acc = __builtin_fmaf(k1, q1, acc);
            }
        }
        red[c] = acc > 0.0f ? acc : 0.0f;
    }
    __syncthreads();
    if (c < R) {
        const int t = t0 + c;
        if (t < a.nq) {
            float s = 0.0f;
            for (int h = 0; h < a.H; ++h) s = s + red[c * a.H + h];
            a.scores[(static_cast<int64_t>(g) * a.nq + t) * a.ld_s + a.b_tail] = s;
        }
    }
}

}  // namespace

hipError_t launch_tail(const ScoreGeom &geo, int64_t b_tail, hipStream_t s) {
    if (geo.nq <= 0 || geo.G <= 0) return hipSuccess;
    const int R = 256 / geo.H;   // H <= 16, so R >= 16
    const int64_t gx = (geo.nq + R - 1) / R;
    if (gx > 0x7fffffffLL || geo.G > 65535) return hipErrorInvalidConfiguration;
    TailArgs a{geo.q16, geo.qts, geo.kblk, geo.khs, geo.scores, geo.ld_s,
               geo.G, geo.nq, geo.H, b_tail, R};
    void *args[] = {&a};
    const void *fn = geo.D == 64 ? reinterpret_cast<const void *>(&tail_kernel<64>)
                                 : reinterpret_cast<const void *>(&tail_kernel<128>);
    return hipLaunchKernel(fn, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(geo.G)),
                           dim3(256), args, 0, s);
}

}  // namespace qsa
