// qsa_tail.hip -- the separate scorer of the partial last KV block.
//
// The pages score the block holding the last n_kv mod bs tokens with its own
// shared kernel whose result is bitwise reproducible (Strata pull request
// #228, part 1, the paragraph naming the tail kernel; pull request #856,
// "What").  Here its order is fixed by construction, per (query, KV head):
//   acc_h = +0;  for i ascending: acc_h = fma(k[i], q_h[i], acc_h)   (fp32)
//   r_h   = acc_h > 0 ? acc_h : +0
//   s     = +0;  for h ascending: s = s + r_h
//   s     = s + 1e9 under the forced-tail rule (Strata pull request #856,
//           "What": the tail keeps its +1e9 rule), which puts the block
//           holding the newest tokens first in every row's selection
// One lane runs one (query, head) chain.  The queries are read once,
// coalesced, and staged through LDS so that every lane walks its own row; a
// second LDS pass sums the heads of each query in order.  HBM-bound: it
// reads 2*H*D bytes per query row.
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
    int32_t G, nq;
    int64_t b_tail;
    int64_t n_items;   // ceil(nq / R) * G
    float tail_add;    // added after the head sum when nonzero
};

// One wave per workgroup: R = 64 / H query rows of one KV head, one lane per
// (row, head) chain.  Work item w covers rows [R*(w/G), R*(w/G)+R) of KV
// head w%G: KV head fastest, so the G items of one row group run side by
// side and together read R whole query rows (G*H*D contiguous fp16 each).
// A workgroup walks items with stride gridDim.x and keeps the next item's
// 16-byte loads in flight (in registers) while it scores the current one
// out of LDS, where each chain is one padded row of D fp16 (pitch D/8 + 1
// chunks: conflict-free 16-byte reads).
template <int D, int H>
__global__ __launch_bounds__(64) void tail_kernel(TailArgs a) {
    constexpr int C8 = D / 8;            // 16-byte chunks per chain
    constexpr int PITCH = C8 + 1;
    constexpr int R = 64 / H;            // query rows per item
    constexpr int HC8 = H * C8;          // chunks per query row
    constexpr int TOTAL = R * HC8;       // chunks per item, <= 64 * C8
    constexpr int PER_LANE = (TOTAL + 63) / 64;
    __shared__ uint4 qs[R * H * PITCH];
    __shared__ uint4 ks[C8];
    __shared__ float red[64];

    const int lane = threadIdx.x;
    // The item's queries (v) and its KV head's tail key (kv, lanes < D/8)
    // travel together: one wait covers both before they are staged in LDS.
    uint4 v[PER_LANE];
    uint4 kv;
    auto fetch = [&](int64_t w) {
        const int g = static_cast<int>(w % a.G);
        const int64_t t0 = w / a.G * R;
        const uint16_t *qg = a.q16 + static_cast<int64_t>(g) * H * D;
        kv = make_uint4(0, 0, 0, 0);
        if (lane < C8)
            kv = *reinterpret_cast<const uint4 *>(a.kblk + static_cast<int64_t>(g) * a.khs +
                                                  a.b_tail * D + 8 * lane);
        #pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int u = lane + 64 * i;
            const int64_t t = t0 + u / HC8;
            v[i] = make_uint4(0, 0, 0, 0);
            if (u < TOTAL && t < a.nq)
                v[i] = *reinterpret_cast<const uint4 *>(qg + t * a.qts + 8 * (u % HC8));
        }
    };

    int64_t w = blockIdx.x;
    if (w < a.n_items) fetch(w);
    for (; w < a.n_items; w += gridDim.x) {
        #pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int u = lane + 64 * i;
            if (u < TOTAL) {
                const int rho = u / HC8, wv = u % HC8;
                qs[(rho * H + wv / C8) * PITCH + wv % C8] = v[i];
            }
        }
        if (lane < C8) ks[lane] = kv;
        __syncthreads();
        const int64_t wn = w + gridDim.x;
        if (wn < a.n_items) fetch(wn);

        const int g = static_cast<int>(w % a.G);
        const int64_t t0 = w / a.G * R;
        if (lane < R * H) {
            float acc = 0.0f;
            #pragma unroll
            for (int j = 0; j < C8; ++j) {
                const uint4 qv = qs[lane * PITCH + j];
                const uint4 kj = ks[j];
                const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                const uint32_t kw[4] = {kj.x, kj.y, kj.z, kj.w};
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
            red[lane] = acc > 0.0f ? acc : 0.0f;
        }
        __syncthreads();
        if (lane < R) {
            const int64_t t = t0 + lane;
            if (t < a.nq) {
                float s = 0.0f;
                #pragma unroll
                for (int h = 0; h < H; ++h) s = s + red[lane * H + h];
                if (a.tail_add != 0.0f) s = s + a.tail_add;
                a.scores[(static_cast<int64_t>(g) * a.nq + t) * a.ld_s + a.b_tail] = s;
            }
        }
        __syncthreads();   // qs and red are rewritten for the next item
    }
}

constexpr int64_t kTailGrid = 2048;

typedef void (*tail_fn)(TailArgs);

template <int D>
tail_fn pick_h(int H) {
    switch (H) {
#define QSA_TAIL_CASE(N) case N: return tail_kernel<D, N>;
        QSA_TAIL_CASE(1) QSA_TAIL_CASE(2) QSA_TAIL_CASE(3) QSA_TAIL_CASE(4)
        QSA_TAIL_CASE(5) QSA_TAIL_CASE(6) QSA_TAIL_CASE(7) QSA_TAIL_CASE(8)
        QSA_TAIL_CASE(9) QSA_TAIL_CASE(10) QSA_TAIL_CASE(11) QSA_TAIL_CASE(12)
        QSA_TAIL_CASE(13) QSA_TAIL_CASE(14) QSA_TAIL_CASE(15) QSA_TAIL_CASE(16)
#undef QSA_TAIL_CASE
    }
    return nullptr;
}

}  // namespace

hipError_t launch_tail(const ScoreGeom &geo, int64_t b_tail, hipStream_t s) {
    if (geo.nq <= 0 || geo.G <= 0) return hipSuccess;
    const int R = 64 / geo.H;   // H <= 16, so R >= 4
    const int64_t items = (geo.nq + R - 1) / R * geo.G;
    // Enough single-wave workgroups to fill every CU several times over; each
    // then walks a few items with the next one's loads in flight.
    const int64_t gx = items < kTailGrid ? items : kTailGrid;
    tail_fn fn = geo.D == 64 ? pick_h<64>(geo.H) : pick_h<128>(geo.H);
    if (!fn) return hipErrorInvalidValue;
    TailArgs a{geo.q16, geo.qts, geo.kblk, geo.khs, geo.scores, geo.ld_s, geo.G, geo.nq, b_tail, items,
                geo.tail_add};
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn),
                           dim3(static_cast<unsigned>(gx)), dim3(64),
                           args, 0, s);
}

}  // namespace qsa
