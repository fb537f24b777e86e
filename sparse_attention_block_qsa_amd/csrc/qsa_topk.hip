// qsa_topk.hip -- per-row top-k block selection of the QSA select phase
// ("selection/topk", Strata pull request #228, part 1; ids compared across
// arms in pull request #856).
//
// Order: score descending, block id ascending on ties; scores compare
// numerically (-0 == +0) and NaN ranks below every number.  This is encoded
// in a 32-bit order key (larger = better): NaN -> 0, -0 -> +0, then the usual
// sign-magnitude flip.  Ids beyond the row also get key 0 and, having the
// largest ids, rank after every real entry.
//
// One wave64 per row, the row's keys held in registers (NPL per lane, block
// id = j*64 + lane), or re-read per pass when the row is longer than the
// register budget.  Steps:
//   1. T = the k-th largest key: a 32-step bisection whose counts are wave
//      ballots + popcounts (no LDS, no atomics);
//   2. the winners are every key > T plus the lowest-id keys == T, taken in
//      id order with ballot prefix ranks (mbcnt);
//   3. the <= 64 winners are compacted into a per-wave LDS slot (64 x 8 bytes,
//      independent of the row length) as (key, ~id) 64-bit composites;
//   4. a bitonic sort across the 64 lanes puts them in order; lane j writes
//      slot j.
#include "qsa_internal.h"

namespace qsa {
namespace {

struct TopkArgs {
    const float *scores;
    int64_t ld_s;
    int32_t *ids;
    int64_t ld_ids;
    float *vals;
    int64_t total_rows, rows_per_group, src_group_rows, dst_group_rows, dst_row0;
    int32_t nb, k;
};

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;   // NaN: lowest
    if (u == 0x80000000u) u = 0u;                      // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const uint32_t plo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), m));
    const uint32_t phi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), m));
    return (static_cast<uint64_t>(phi) << 32) | plo;
}

// NPL > 0: keys held in registers (row length <= 64*NPL).
// NPL == 0: keys recomputed from memory in every pass (any row length).
template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
    __shared__ uint64_t slot[4][64];
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t R = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (R >= a.total_rows) return;               // whole wave; no block barriers below
    const int64_t grp = R / a.rows_per_group, t = R % a.rows_per_group;
    const float *srow = a.scores + (grp * a.src_group_rows + t) * a.ld_s;
    const int64_t drow = grp * a.dst_group_rows + a.dst_row0 + t;
    const int nb = a.nb;
    const int kk = min(a.k, nb);
    const int nj = (nb + 63) >> 6;               // 64-wide columns of the row
    const uint64_t lt = (1ull << lane) - 1ull;

    uint32_t kr[NPL > 0 ? NPL : 1];
    if constexpr (NPL > 0) {
        #pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int id = j * 64 + lane;
            kr[j] = id < nb ? order_key(srow[id]) : 0u;
        }
    }
    auto key = [&](int j) -> uint32_t {
        if constexpr (NPL > 0) {
            return kr[j];
        } else {
            const int id = j * 64 + lane;
            return id < nb ? order_key(srow[id]) : 0u;
        }
    };
    const int jmax = NPL > 0 ? NPL : nj;   // a constant when keys are in registers

    uint64_t v = 0;
    if (kk > 0) {
        // 1. bisection for T = max { x : #(key >= x) >= kk }
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
            #pragma unroll
            for (int j = 0; j < jmax; ++j) cnt += __popcll(ballot(key(j) >= cand));
            if (cnt >= kk) T = cand;
        }
        // 2-3. winners: key > T, then ties at T in id order
        int cgt = 0;
        for (int j = 0; j < jmax; ++j) cgt += __popcll(ballot(key(j) > T));
        int need = kk - cgt;
        int base = 0;
        for (int j = 0; j < jmax; ++j) {
            const uint32_t kj = key(j);
            const int id = j * 64 + lane;
            const bool eq = (kj == T) && (id < nb);
            const uint64_t meq = ballot(eq);
            const bool tsel = eq && (__popcll(meq & lt) < need);
            const int ceq = __popcll(meq);
            need -= ceq < need ? ceq : need;
            const bool sel = (kj > T) || tsel;
            const uint64_t ms = ballot(sel);
            if (sel)
                slot[w][base + __popcll(ms & lt)] =
                    (static_cast<uint64_t>(kj) << 32) | (0xffffffffu - static_cast<uint32_t>(id));
            base += __popcll(ms);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        v = lane < kk ? slot[w][lane] : 0ull;

        // 4. bitonic sort, descending, across the 64 lanes
        #pragma unroll
        for (int size = 2; size <= 64; size <<= 1) {
            #pragma unroll
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                const uint64_t p = shfl_xor_u64(v, stride);
                const bool lower = (lane & stride) == 0;
                const bool first_half_dir = (lane & size) == 0;
                const bool keep_max = (lower == first_half_dir);
                v = keep_max ? (v > p ? v : p) : (v < p ? v : p);
            }
        }
    }

    if (lane < a.k) {
        int32_t id = -1;
        float val = -__builtin_inff();
        if (lane < kk) {
            id = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(v));
            val = srow[id];
        }
        a.ids[drow * a.ld_ids + lane] = id;
        if (a.vals) a.vals[drow * a.ld_ids + lane] = val;
    }
}

typedef void (*topk_fn)(TopkArgs);

topk_fn pick(int nb, int *npl_out) {
    const int nj = (nb + 63) / 64;
#define QSA_TOPK_CASE(N) \
    if (nj <= N) { *npl_out = N; return topk_kernel<N>; }
    QSA_TOPK_CASE(1)
    QSA_TOPK_CASE(2)
    QSA_TOPK_CASE(4)
    QSA_TOPK_CASE(8)
    QSA_TOPK_CASE(16)
    QSA_TOPK_CASE(24)
    QSA_TOPK_CASE(32)
    QSA_TOPK_CASE(33)
    QSA_TOPK_CASE(40)
    QSA_TOPK_CASE(48)
    QSA_TOPK_CASE(64)
#undef QSA_TOPK_CASE
    *npl_out = 0;
    return topk_kernel<0>;
}

}  // namespace

hipError_t launch_topk(const TopkGeom &geo, hipStream_t s) {
    const int64_t total = geo.n_groups * geo.rows_per_group;
    if (total <= 0 || geo.k <= 0) return hipSuccess;
    const int64_t blocks = (total + 3) / 4;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    TopkArgs a{geo.scores, geo.ld_s, geo.ids, geo.ld_ids, geo.vals, total,
               geo.rows_per_group, geo.src_group_rows, geo.dst_group_rows, geo.dst_row0,
               geo.nb, geo.k};
    int npl = 0;
    topk_fn fn = pick(geo.nb, &npl);
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(static_cast<unsigned>(blocks)),
                           dim3(256), args, 0, s);
}

}  // namespace qsa
