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
// a sampled threshold filters the row down to <= 128 candidates, whose exact
// composites are sorted by a bitonic network (see topk_kernel); rows the
// filter cannot reduce take an exact ballot-bisection path.  LDS use is a
// per-wave slot of 128 x 8 bytes, independent of the row length.
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

// Sorting networks in the uniform-direction (mirror) form of the bitonic
// sort: every compare-exchange keeps the larger composite at the lower
// element index, so the only per-lane input is whether this lane holds the
// lower element of its pair.  Merge of size s: first partner e ^ (s-1), then
// partners e ^ (s/4), ..., e ^ 1.
__device__ __forceinline__ uint64_t cx_keep(uint64_t v, uint64_t p, bool lower) {
    return ((p > v) == lower) ? p : v;   // lower keeps max, upper keeps min
}

// 128 composites held two per lane (element e = s*64 + lane), descending:
// afterwards slot 0 of lanes 0..63 holds the 64 largest in order.
__device__ __forceinline__ void bitonic128_desc(uint64_t &v0, uint64_t &v1, int lane) {
    #pragma unroll
    for (int size = 2; size <= 128; size <<= 1) {
        if (size == 128) {
            // mirror across the slots: element lane pairs with 127 - lane,
            // which is slot 1 of lane ^ 63
            const uint64_t p0 = shfl_xor_u64(v1, 63);
            const uint64_t p1 = shfl_xor_u64(v0, 63);
            v0 = cx_keep(v0, p0, true);
            v1 = cx_keep(v1, p1, false);
        } else {
            const bool lower = (lane & (size >> 1)) == 0;
            v0 = cx_keep(v0, shfl_xor_u64(v0, size - 1), lower);
            v1 = cx_keep(v1, shfl_xor_u64(v1, size - 1), lower);
        }
        #pragma unroll
        for (int stride = size >> 2; stride > 0; stride >>= 1) {
            const bool lower = (lane & stride) == 0;
            v0 = cx_keep(v0, shfl_xor_u64(v0, stride), lower);
            v1 = cx_keep(v1, shfl_xor_u64(v1, stride), lower);
        }
    }
}

__device__ __forceinline__ uint64_t bitonic64_desc(uint64_t v, int lane) {
    #pragma unroll
    for (int size = 2; size <= 64; size <<= 1) {
        v = cx_keep(v, shfl_xor_u64(v, size - 1), (lane & (size >> 1)) == 0);
        #pragma unroll
        for (int stride = size >> 2; stride > 0; stride >>= 1)
            v = cx_keep(v, shfl_xor_u64(v, stride), (lane & stride) == 0);
    }
    return v;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int id) {
    return (static_cast<uint64_t>(key) << 32) | (0xffffffffu - static_cast<uint32_t>(id));
}

// Exclusive prefix sum over the wave.
__device__ __forceinline__ int wave_excl_scan(int x, int lane, int *total) {
    int incl = x;
    #pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    *total = __shfl(incl, 63);
    return incl - x;
}

// NPL > 0: the row's values held in registers (row length <= 64*NPL).
// NPL == 0: values re-read from memory in every pass (any row length).
//
// Fast path (NPL > 0).  A threshold th is sampled from the per-lane top two
// values (ordered as signed integers of the fp32 bits, exact for scores >= 0,
// merely a heuristic otherwise), and the candidates are the values x >= th
// (an fp32 compare: NaN never qualifies, -0 == +0).  If their number C
// satisfies kk <= C <= 128, every element of the true top-kk is a candidate
// (kk elements are >= th, so the kk-th largest is too), whatever th was; the
// candidates' exact (key, ~id) composites are compacted into LDS and sorted
// by a 128-wide bitonic network.  Any other C takes the exact path: a 32-step
// ballot bisection for the kk-th largest key over every value, then ties in
// id order.
template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
    __shared__ uint64_t slot[4][128];
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t R = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (R >= a.total_rows) return;               // whole wave; no block barriers below
    int64_t grp = 0, t = R;
    if (a.rows_per_group != a.total_rows) {   // grouped rows (the phase's chunks)
        grp = R / a.rows_per_group;
        t = R - grp * a.rows_per_group;
    }
    const float *srow = a.scores + (grp * a.src_group_rows + t) * a.ld_s;
    const int64_t drow = grp * a.dst_group_rows + a.dst_row0 + t;
    const int nb = a.nb;
    const int kk = min(a.k, nb);
    const int nj = (nb + 63) >> 6;               // 64-wide columns of the row
    const uint64_t lt = (1ull << lane) - 1ull;
    // Padding past the row: a NaN (never >= a threshold) whose bits, read as
    // a signed integer (-1), rank above every negative float and below every
    // non-negative one.
    const uint32_t kPad = 0xffffffffu;

    uint32_t xr[NPL > 0 ? NPL : 1];              // raw fp32 bits
    if constexpr (NPL > 0) {
        #pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const int id = j * 64 + lane;
            xr[j] = id < nb ? __builtin_bit_cast(uint32_t, srow[id]) : kPad;
        }
    }
    auto key = [&](int j) -> uint32_t {
        const int id = j * 64 + lane;
        if constexpr (NPL > 0) {
            return id < nb ? order_key(__builtin_bit_cast(float, xr[j])) : 0u;
        } else {
            return id < nb ? order_key(srow[id]) : 0u;
        }
    };
    const int jmax = NPL > 0 ? NPL : nj;   // a constant when values are in registers

    uint64_t v = 0;
    bool done = false;
    if constexpr (NPL > 0) {
        if (kk > 0) {
            // 1. per-lane top two of the fp32 bits as signed integers
            int32_t m1 = INT32_MIN, m2 = INT32_MIN;
            #pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const int32_t x = static_cast<int32_t>(xr[j]);
                m2 = max(m2, min(m1, x));
                m1 = max(m1, x);
            }
            // 2. th = the kk-th largest of the 128 samples (bisection on the
            //    biased bits, two ballots per step)
            const uint32_t s1 = static_cast<uint32_t>(m1) ^ 0x80000000u;
            const uint32_t s2 = static_cast<uint32_t>(m2) ^ 0x80000000u;
            uint32_t T = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                const int cnt = __popcll(ballot(s1 >= cand)) + __popcll(ballot(s2 >= cand));
                if (cnt >= kk) T = cand;
            }
            const float th = __builtin_bit_cast(float, T ^ 0x80000000u);
            // 3. candidates x >= th as a per-lane bitmask over j
            uint32_t mlo = 0, mhi = 0;
            #pragma unroll
            for (int j = 0; j < NPL; ++j) {
                const bool c = __builtin_bit_cast(float, xr[j]) >= th;
                if (j < 32) mlo |= static_cast<uint32_t>(c) << j;
                else mhi |= static_cast<uint32_t>(c) << (j - 32);
            }
            const int cnt = __popc(mlo) + __popc(mhi);
            int C = 0;
            int off = wave_excl_scan(cnt, lane, &C);
            if (C >= kk && C <= 128) {
                // 4. compact the candidates' exact composites into LDS: up to
                //    four per lane per round, their reloads issued together
                uint64_t more = ballot(cnt > 0);
                while (more) {
                    int id4[4];
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        id4[r] = -1;
                        if (mlo | mhi) {
                            const int j = mlo ? __builtin_ctz(mlo) : 32 + __builtin_ctz(mhi);
                            if (mlo) mlo &= mlo - 1; else mhi &= mhi - 1;
                            id4[r] = j * 64 + lane;
                        }
                    }
                    float x4[4];
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) x4[r] = id4[r] >= 0 ? srow[id4[r]] : 0.0f;
                    #pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (id4[r] >= 0) slot[w][off++] = composite(order_key(x4[r]), id4[r]);
                    more = ballot((mlo | mhi) != 0);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                uint64_t v0 = lane < C ? slot[w][lane] : 0ull;
                uint64_t v1 = lane + 64 < C ? slot[w][lane + 64] : 0ull;
                bitonic128_desc(v0, v1, lane);
                v = v0;
                done = true;
            }
        }
    }

    if (kk > 0 && !done) {
        // exact path: T = max { x : #(key >= x) >= kk }
        uint32_t T = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            int cnt = 0;
            #pragma unroll (NPL > 0 ? NPL : 1)
            for (int j = 0; j < jmax; ++j) cnt += __popcll(ballot(key(j) >= cand));
            if (cnt >= kk) T = cand;
        }
        // winners: key > T, then ties at T in id order
        int cgt = 0;
        #pragma unroll (NPL > 0 ? NPL : 1)
        for (int j = 0; j < jmax; ++j) cgt += __popcll(ballot(key(j) > T));
        int need = kk - cgt;
        int base = 0;
        #pragma unroll (NPL > 0 ? NPL : 1)
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
            if (sel) slot[w][base + __popcll(ms & lt)] = composite(kj, id);
            base += __popcll(ms);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        v = bitonic64_desc(lane < kk ? slot[w][lane] : 0ull, lane);
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
