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
// Every form takes the same steps: a sampled threshold filters the row down
// to <= 128 candidates, whose exact composites are sorted by bitonic networks
// over the wave's lanes; a row the filter cannot reduce takes an exact
// ballot-bisection path.  The row's values are also stashed in LDS, so that a
// candidate's value is read back by id.  Launch forms:
//  * topk_kernel<NPL, MANY>: one wave64 per row, the row's values held in
//    registers (NPL per lane, block id = j*64 + lane), or re-read per pass
//    past the register budget (NPL = 0).  One row per workgroup for few rows;
//    four per workgroup for many (MANY), where VALU throughput rather than a
//    row's latency bounds the launch and the steps with fewer ops are taken.
//  * topk_quad_kernel<NC>: few rows of more than 512 blocks, four waves per
//    row, the waves' candidates pooled into one set.
#include "qsa_topk_row.h"

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

// R / rows_per_group for a wave-uniform row R: a 32-bit division (a few
// scalar ops) when the rows fit in 31 bits, else the 64-bit one (about 190).
__device__ __forceinline__ int64_t row_group(int64_t R, int64_t rows_per_group, int64_t total_rows) {
    if (total_rows <= 0x7fffffff)   // uniform
        return static_cast<uint32_t>(R) / static_cast<uint32_t>(rows_per_group);
    return R / rows_per_group;
}

template <int NPL, bool MANY>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
    __shared__ uint64_t slot[4][128];   // one per wave of the workgroup (at most four)
    __shared__ uint32_t stash[4][NPL > 0 ? 64 * NPL : 1];   // the row's values, per wave
    // the wave index is uniform over the wave: say so, so that the row's
    // addresses and buffer descriptor live in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    // rows in the scorers' XCD order: row R is read on the XCD that wrote it
    const int64_t R = static_cast<int64_t>(xcd_logical_id(blockIdx.x, gridDim.x)) * (blockDim.x >> 6) + w;
    if (R >= a.total_rows) return;               // whole wave; no block barriers below
    int64_t grp = 0, t = R;
    if (a.rows_per_group != a.total_rows) {   // grouped rows (the phase's chunks)
        grp = row_group(R, a.rows_per_group, a.total_rows);
        t = R - grp * a.rows_per_group;
    }
    const float *srow = a.scores + (grp * a.src_group_rows + t) * a.ld_s;
    const int64_t drow = grp * a.dst_group_rows + a.dst_row0 + t;
    uint32_t xr[NPL > 0 ? NPL : 1];
    topk_row_load<NPL>(srow, a.nb, lane, xr);
    topk_row_select<NPL, MANY>(srow, a.nb, a.k, xr, a.ids + drow * a.ld_ids,
                               a.vals ? a.vals + drow * a.ld_ids : nullptr, slot[w], stash[w],
                               lane);
}

// A threshold from the per-lane top two of NC columns held by one wave
// (fp32 bits ordered as signed integers, exact for scores >= 0, merely a
// heuristic otherwise): the kq-th largest of those 128 samples, to 16 leading
// bits (bisection on the biased bits, two ballots per step), as biased bits.
// Any threshold is correct for the callers, who check the count they get.
template <int NC>
__device__ __forceinline__ uint32_t sampled_threshold(const uint32_t (&xr)[NC], int kq) {
    int32_t m1 = INT32_MIN, m2 = INT32_MIN;
    #pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int32_t x = static_cast<int32_t>(xr[j]);
        m2 = max(min(m1, x), min(max(m1, x), m2));   // median of three: v_med3_i32
        m1 = max(m1, x);
    }
    const uint32_t s1 = static_cast<uint32_t>(m1) ^ 0x80000000u;
    const uint32_t s2 = static_cast<uint32_t>(m2) ^ 0x80000000u;
    uint32_t T = 0;
    for (int bit = 31; bit >= 16; --bit) {
        const uint32_t cand = T | (1u << bit);
        const int c = __popcll(ballot(s1 >= cand)) + __popcll(ballot(s2 >= cand));
        if (c >= kq) T = cand;
    }
    return T;
}

// The exact top-kk (kk <= 64) of NC 64-wide columns of values held by one
// wave (column jj of this wave is column col0 + jj of the row, block id
// (col0 + jj)*64 + lane; ids at or past id_end are padding, NaN in xr), or
// all of them when the wave holds fewer than kk, returned as composites
// sorted descending over the lanes (lane 0 largest, zero past the set).  The same steps as topk_kernel's fast path (sampled
// threshold, candidates compacted into slot, bitonic sort) with its exact
// bisection as the fallback; val(id) reads a value back by id.
template <int NC, typename Val>
__device__ __forceinline__ uint64_t wave_topk(const uint32_t (&xr)[NC], int col0, int kk, int id_end,
                                              int lane, uint64_t *slot, Val val) {
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t T = sampled_threshold<NC>(xr, kk);
    const float th = __builtin_bit_cast(float, T ^ 0x80000000u);
    uint32_t mask = 0;
    #pragma unroll
    for (int j = 0; j < NC; ++j)
        mask |= static_cast<uint32_t>(__builtin_bit_cast(float, xr[j]) >= th) << j;
    int C = 0;
    int off = wave_excl_scan(__popc(mask), lane, &C);
    if (C >= kk && C <= 128) {
        while (mask) {
            const int j = __builtin_ctz(mask);
            mask &= mask - 1;
            const int id = (col0 + j) * 64 + lane;
            slot[off++] = composite(order_key(val(id)), id);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        return sorted_top64(slot, C, order_key(th), lane, false);
    }
    // exact path over the wave's columns
    auto key = [&](int j) -> uint32_t { return order_key(__builtin_bit_cast(float, xr[j])); };
    T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int c = 0;
        #pragma unroll
        for (int j = 0; j < NC; ++j) c += __popcll(ballot(key(j) >= cand));
        if (c >= kk) T = cand;
    }
    int cgt = 0;
    #pragma unroll
    for (int j = 0; j < NC; ++j) cgt += __popcll(ballot(key(j) > T));
    int need = kk - cgt;
    int base = 0;
    #pragma unroll
    for (int j = 0; j < NC; ++j) {
        const uint32_t kj = key(j);
        const int id = (col0 + j) * 64 + lane;
        const bool eq = (kj == T) && (id < id_end);
        const uint64_t meq = ballot(eq);
        const bool tsel = eq && (__popcll(meq & lt) < need);
        const int ceq = __popcll(meq);
        need -= ceq < need ? ceq : need;
        const bool sel = (kj > T) || tsel;
        const uint64_t ms = ballot(sel);
        if (sel) slot[base + __popcll(ms & lt)] = composite(kj, id);
        base += __popcll(ms);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // base < kk when the wave holds fewer than kk of the row's values (a short
    // or empty last wave): only the slots written are read
    return sort64_desc(lane < base ? slot[lane] : 0ull, lane);
}

// Two composite lists, each sorted descending over the lanes: the 64 largest
// of their union, sorted descending (the first merge step pairs element i of
// one with element 63 - i of the other; the larger halves form a bitonic
// sequence, which the half-cleaner cascade sorts).
__device__ __forceinline__ uint64_t merge64(uint64_t v, uint64_t u_rev, int lane) {
    uint64_t m = v > u_rev ? v : u_rev;
    step1<32, 32>(m, lane);
    step1<16, 16>(m, lane);
    step1<8, 8>(m, lane);
    step1<4, 4>(m, lane);
    step1<2, 2>(m, lane);
    step1<1, 1>(m, lane);
    return m;
}

// Few rows of more than 512 blocks (latency-bound): one workgroup of four
// waves per row.  The row's ncol columns are shared out evenly, wave w
// holding columns [w*ncol/4, (w+1)*ncol/4), at most NC of them: with the
// values spread alike the four sampled thresholds below are alike too.
//
// Pooled path.  Wave w, holding nw of the row's nb values, samples a
// threshold that at least ceil(kk*nw/nb) of its values reach.  These shares
// sum to at least kk, so the smallest of the four thresholds is one that at
// least kk values of the row reach; shares in proportion to the values keep
// the pool near kk.  The waves compact the candidates x >= th into one pool
// (offsets from an LDS counter), and if it holds kk..128 of them the row's
// top-kk is among them: wave 0 sorts a pool of up to 64, and a fuller one is
// sorted half by wave 0 and half by wave 1, then merged by wave 0.
//
// Otherwise each wave finds the exact top-kk of its own columns (wave_topk);
// the union of the four holds the row's top-kk, and two levels of merge64
// give it sorted.
template <int NC>
__global__ __launch_bounds__(256) void topk_quad_kernel(TopkArgs a) {
    __shared__ uint32_t row[4 * NC * 64];        // the row's raw fp32 bits (pad past nb)
    __shared__ uint64_t slot[4][128];            // per-wave slots; slot[0] is also the pool
    __shared__ uint64_t lists[4][64];
    __shared__ uint32_t thr[4];
    __shared__ int pool_n;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    // rows in the scorers' XCD order: row R is read on the XCD that wrote it
    const int64_t R = xcd_logical_id(blockIdx.x, gridDim.x);
    if (R >= a.total_rows) return;               // whole workgroup
    int64_t grp = 0, t = R;
    if (a.rows_per_group != a.total_rows) {
        grp = row_group(R, a.rows_per_group, a.total_rows);
        t = R - grp * a.rows_per_group;
    }
    const float *srow = a.scores + (grp * a.src_group_rows + t) * a.ld_s;
    const int64_t drow = grp * a.dst_group_rows + a.dst_row0 + t;
    const int nb = a.nb;
    const int kk = min(a.k, nb);
    const uint32_t kPad = 0xffffffffu;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(srow), 0, nb * 4, 0x00020000 /* 32-bit elements, raw */);
    const int ncol = (nb + 63) >> 6;
    const int col0 = w * ncol / 4, ncw = (w + 1) * ncol / 4 - col0;   // this wave's columns
    const int id_end = min(nb, (col0 + ncw) * 64);                    // ... and its ids
    const int nw = max(id_end - col0 * 64, 0);                        // ... and its values
    uint32_t xr[NC];
    #pragma unroll
    for (int j = 0; j < NC; ++j) {
        // All NC columns are loaded and stashed: a column past the share is
        // the next wave's, which stashes the same bits, or lies past nb
        // (pads, never read back).  Ownership is a per-lane test, so that
        // no load or store sits under a branch that would serialise them.
        const int c = col0 + j;
        const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, c * 256, 0);
        const uint32_t xv = lane < nb - 64 * c ? x : kPad;
        row[c * 64 + lane] = xv;
        xr[j] = 64 * j + lane < nw ? xv : kPad;
    }
    if (threadIdx.x == 0) pool_n = 0;
    uint64_t v = 0;
    bool pooled = false;
    if (kk > 0) {   // uniform
        // a share of kk proportional to the wave's values; the shares sum to >= kk
        const uint32_t Tw = sampled_threshold<NC>(xr, (kk * nw + nb - 1) / nb);
        if (lane == 0) thr[w] = Tw;
        __syncthreads();   // also publishes the row stash and the zeroed counter
        const uint32_t T = min(min(thr[0], thr[1]), min(thr[2], thr[3]));
        const float th = __builtin_bit_cast(float, T ^ 0x80000000u);
        uint32_t mask = 0;
        #pragma unroll
        for (int j = 0; j < NC; ++j)
            mask |= static_cast<uint32_t>(__builtin_bit_cast(float, xr[j]) >= th) << j;
        int cw = 0;
        int off = wave_excl_scan(__popc(mask), lane, &cw);
        int base = 0;
        if (lane == 0 && cw > 0) base = atomicAdd(&pool_n, cw);
        base = __builtin_amdgcn_readfirstlane(base);
        if (base + cw <= 128) {   // uniform; a fuller pool is not used
            off += base;
            while (mask) {
                const int j = __builtin_ctz(mask);
                mask &= mask - 1;
                const int id = (col0 + j) * 64 + lane;
                slot[0][off++] = composite(order_key(__builtin_bit_cast(float, row[id])), id);
            }
        }
        __syncthreads();
        const int C = pool_n;   // uniform over the workgroup
        pooled = C >= kk && C <= 128;
        if (pooled) {   // uniform over the workgroup
            if (C > 64) {
                // waves 0 and 1 sort the pool's two halves side by side and
                // wave 0 merges them: one 64-wide sort and a merge on the
                // row's path instead of the 128 -> 64 network on one wave
                if (w == 1) lists[1][lane] = sort64_desc(lane + 64 < C ? slot[0][lane + 64] : 0ull, lane);
                if (w == 0) v = sort64_desc(slot[0][lane], lane);
                __syncthreads();   // every wave, so that no barrier counts on ended waves
                if (w != 0) return;
                v = merge64(v, lists[1][63 - lane], lane);
            } else {
                if (w != 0) return;
                v = sort64_desc(lane < C ? slot[0][lane] : 0ull, lane);
            }
        }
    }
    if (!pooled) {   // uniform
        if (kk > 0) {
            v = wave_topk<NC>(xr, col0, kk, id_end, lane, slot[w],
                              [&](int id) { return __builtin_bit_cast(float, row[id]); });
            lists[w][lane] = v;
        }
        __syncthreads();
        if (kk > 0 && (w & 1) == 0) {   // waves 0, 2: merge with wave w + 1
            v = merge64(v, lists[w + 1][63 - lane], lane);
            lists[w][lane] = v;
        }
        __syncthreads();
        if (w != 0) return;
        if (kk > 0) v = merge64(v, lists[2][63 - lane], lane);
    }
    if (lane < a.k) {
        int32_t id = -1;
        float val = -__builtin_inff();
        if (lane < kk) {
            id = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(v));
            val = __builtin_bit_cast(float, row[id]);
        }
        a.ids[drow * a.ld_ids + lane] = id;
        if (a.vals) a.vals[drow * a.ld_ids + lane] = val;
    }
}

typedef void (*topk_fn)(TopkArgs);

// The first case of the table that holds nj columns (topk_kernel<0, .>, the
// re-reading path, past the last).
template <bool MANY, int I = 0>
topk_fn pick_case(int nj, int *npl_out) {
    constexpr int kN = sizeof(kTopkCases) / sizeof(kTopkCases[0]);
    if constexpr (I < kN) {
        constexpr int N = kTopkCases[I];
        if (nj <= N) {
            *npl_out = N;
            return topk_kernel<N, MANY>;
        }
        return pick_case<MANY, I + 1>(nj, npl_out);
    } else {
        *npl_out = 0;
        return topk_kernel<0, MANY>;
    }
}

// many: the launch of many rows (four per workgroup), which the VALU's
// throughput bounds rather than each row's chain of steps
topk_fn pick(int nb, bool many, int *npl_out) {
    const int nj = (nb + 63) / 64;
    return many ? pick_case<true>(nj, npl_out) : pick_case<false>(nj, npl_out);
}

}  // namespace

hipError_t launch_topk(const TopkGeom &geo, hipStream_t s) {
    const int64_t total = geo.n_groups * geo.rows_per_group;
    if (total <= 0 || geo.k <= 0) return hipSuccess;
    const int ncol = (geo.nb + 63) / 64;
    // Few rows of more than 512 blocks, or of 129..512 blocks with k > 32:
    // four waves per row.  The four waves pay for their barriers when the
    // pool is likely to hold more than 64 candidates, whose sort they split:
    // at nq = 256 and k = 64, 512 blocks 7.78 -> 7.48 us per phase and 256
    // blocks 7.32 -> 7.23 us; at 512 blocks and k = 32 one wave per row stays
    // ahead (7.13 against 7.20 us).
    if (total < 4096 && ncol <= 64 && (ncol > 8 || (ncol > 2 && geo.k > 32))) {
        TopkArgs qa{geo.scores, geo.ld_s, geo.ids, geo.ld_ids, geo.vals, total,
                    geo.rows_per_group, geo.src_group_rows, geo.dst_group_rows, geo.dst_row0,
                    geo.nb, geo.k};
        topk_fn fn = ncol <= 8 ? topk_quad_kernel<2> : ncol <= 16 ? topk_quad_kernel<4>
                   : ncol <= 32 ? topk_quad_kernel<8>
                   : ncol <= 36 ? topk_quad_kernel<9> : ncol <= 48 ? topk_quad_kernel<12>
                                                       : topk_quad_kernel<16>;
        void *qargs[] = {&qa};
        return hipLaunchKernel(reinterpret_cast<const void *>(fn),
                               dim3(static_cast<unsigned>(total)), dim3(256), qargs, 0, s);
    }
    // One row per wave.  Few rows: one wave per workgroup, so that the rows
    // spread over all CUs; many rows: four per workgroup.
    const int wpb = total < 4096 ? 1 : 4;
    const int64_t blocks = (total + wpb - 1) / wpb;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    TopkArgs a{geo.scores, geo.ld_s, geo.ids, geo.ld_ids, geo.vals, total,
               geo.rows_per_group, geo.src_group_rows, geo.dst_group_rows, geo.dst_row0,
               geo.nb, geo.k};
    int npl = 0;
    topk_fn fn = pick(geo.nb, wpb == 4, &npl);
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(static_cast<unsigned>(blocks)),
                           dim3(64 * wpb), args, 0, s);
}

}  // namespace qsa
