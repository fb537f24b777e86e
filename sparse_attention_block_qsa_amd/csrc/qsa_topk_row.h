// qsa_topk_row.h -- the one-wave selection of one score row: the device
// code of the per-row selector in qsa_topk.hip, shared with the scorer's
// fused-selection epilogue in qsa_score.hip ("selection/topk", Strata pull
// request #228, part 1; ids compared across arms in pull request #856).
//
// Order: score descending, block id ascending on ties; scores compare
// numerically (-0 == +0) and NaN ranks below every number.  This is encoded
// in a 32-bit order key (larger = better): NaN -> 0, -0 -> +0, then the usual
// sign-magnitude flip.  Ids beyond the row also get key 0 and, having the
// largest ids, rank after every real entry.
#pragma once

#include "qsa_internal.h"

namespace qsa {
namespace {

__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;   // NaN: lowest
    if (u == 0x80000000u) u = 0u;                      // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// 2*mask + (x >= th) in two VALU ops: the compare writes VCC and the add
// takes it as its carry (written as C, the compiler turns the add into ORs of
// shifted select results, three to four ops).  NaN never compares >= .
__device__ __forceinline__ uint32_t shift_in_ge(uint32_t mask, float x, float th) {
    asm("v_cmp_le_f32 vcc, %2, %1\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
        : "+v"(mask) : "v"(x), "v"(th) : "vcc");
    return mask;
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

// The value of lane ^ M through lane permutations of the VALU: DPP quad
// permutes (xor 1, 2, 3), DPP row mirrors (xor 7 within 8 lanes, xor 15
// within 16), DPP row rotates (xor 8 = rotate by 8; xor 4 = rotate by 4 or
// by 12, picked by lane bit 2), v_permlane16/32_swap (xor 16, xor 32:
// swapping a register with itself exchanges the two row halves), and the
// compositions xor 31 = xor 15 then xor 16, xor 63 = xor 31 then xor 32.
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int lane) {
    if constexpr (M == 4) {
        const uint32_t a = dpp_mov<0x124>(v), b = dpp_mov<0x12C>(v);   // row_ror:4, row_ror:12
        return (lane & 4) ? a : b;
    } else if constexpr (M == 8) {
        return dpp_mov<0x128>(v);                                       // row_ror:8
    } else if constexpr (M == 31) {
        return xor_lane<16>(dpp_mov<0x140>(v), lane);                  // row_mirror, then xor 16
    } else if constexpr (M == 1) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, false));
    } else if constexpr (M == 2) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, false));
    } else if constexpr (M == 3) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x1B, 0xF, 0xF, false));
    } else if constexpr (M == 7) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x141, 0xF, 0xF, false));
    } else if constexpr (M == 15) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x140, 0xF, 0xF, false));
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else if constexpr (M == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    } else {
        static_assert(M == 63, "unsupported lane mask");
        return xor_lane<32>(xor_lane<31>(v, lane), lane);
    }
}

template <int M, typename T>
__device__ __forceinline__ T xor_lane_t(T v, int lane) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit elements");
    if constexpr (sizeof(T) == 4) {
        return static_cast<T>(xor_lane<M>(static_cast<uint32_t>(v), lane));
    } else {
        const uint32_t lo = xor_lane<M>(static_cast<uint32_t>(v), lane);
        const uint32_t hi = xor_lane<M>(static_cast<uint32_t>(v >> 32), lane);
        return static_cast<T>((static_cast<uint64_t>(hi) << 32) | lo);
    }
}

// Compare-exchange with the partner's value p: keep the larger or the smaller.
template <typename T>
__device__ __forceinline__ T cmpx(T v, T p, bool keep_max) {
    return ((p > v) == keep_max) ? p : v;
}

// Bitonic networks in the uniform-direction (mirror) form: a merge of size s
// first pairs element e with its mirror e ^ (s-1), then with e ^ (s/4), ...,
// e ^ 1; the element of the pair with the clear bit keeps the larger value
// (descending) or the smaller (ascending).  One element per lane: a 64-bit
// (key, ~id) composite, or a 32-bit word of the same order.
template <int M, int B, typename T>
__device__ __forceinline__ void step2(T &v0, T &v1, int lane) {
    const T p0 = xor_lane_t<M>(v0, lane);
    const T p1 = xor_lane_t<M>(v1, lane);
    const bool lower = (lane & B) == 0;
    v0 = cmpx(v0, p0, lower);    // descending
    v1 = cmpx(v1, p1, !lower);   // ascending
}
template <int M, int B, typename T>
__device__ __forceinline__ void step1(T &v, int lane) {
    v = cmpx(v, xor_lane_t<M>(v, lane), (lane & B) == 0);
}

// Sorts v0 descending and v1 ascending over the 64 lanes.
template <typename T>
__device__ __forceinline__ void sort64_pair(T &v0, T &v1, int lane) {
    step2<1, 1>(v0, v1, lane);
    step2<3, 2>(v0, v1, lane);   step2<1, 1>(v0, v1, lane);
    step2<7, 4>(v0, v1, lane);   step2<2, 2>(v0, v1, lane);   step2<1, 1>(v0, v1, lane);
    step2<15, 8>(v0, v1, lane);  step2<4, 4>(v0, v1, lane);   step2<2, 2>(v0, v1, lane);
    step2<1, 1>(v0, v1, lane);
    step2<31, 16>(v0, v1, lane); step2<8, 8>(v0, v1, lane);   step2<4, 4>(v0, v1, lane);
    step2<2, 2>(v0, v1, lane);   step2<1, 1>(v0, v1, lane);
    step2<63, 32>(v0, v1, lane); step2<16, 16>(v0, v1, lane); step2<8, 8>(v0, v1, lane);
    step2<4, 4>(v0, v1, lane);   step2<2, 2>(v0, v1, lane);   step2<1, 1>(v0, v1, lane);
}

// Sorts v descending over the 64 lanes (lane 0 largest).
template <typename T>
__device__ __forceinline__ T sort64_desc(T v, int lane) {
    step1<1, 1>(v, lane);
    step1<3, 2>(v, lane);   step1<1, 1>(v, lane);
    step1<7, 4>(v, lane);   step1<2, 2>(v, lane);   step1<1, 1>(v, lane);
    step1<15, 8>(v, lane);  step1<4, 4>(v, lane);   step1<2, 2>(v, lane);   step1<1, 1>(v, lane);
    step1<31, 16>(v, lane); step1<8, 8>(v, lane);   step1<4, 4>(v, lane);   step1<2, 2>(v, lane);
    step1<1, 1>(v, lane);
    step1<63, 32>(v, lane); step1<16, 16>(v, lane); step1<8, 8>(v, lane);   step1<4, 4>(v, lane);
    step1<2, 2>(v, lane);   step1<1, 1>(v, lane);
    return v;
}

// The 64 largest of 128 elements (two per lane), sorted descending: sort
// the slots in opposite directions, so that element i of the 128-sequence
// meets element i + 64 in the same lane; the larger of each pair forms a
// bitonic sequence holding the 64 largest, which a half-cleaner cascade
// (partners lane ^ 32, ..., lane ^ 1) sorts.  *rest receives the smaller of
// each pair: the 64 elements left out.
template <typename T>
__device__ __forceinline__ T top64_of_128(T v0, T v1, int lane, T *rest = nullptr) {
    sort64_pair(v0, v1, lane);
    T v = v0 > v1 ? v0 : v1;
    if (rest) *rest = v0 > v1 ? v1 : v0;
    step1<32, 32>(v, lane);
    step1<16, 16>(v, lane);
    step1<8, 8>(v, lane);
    step1<4, 4>(v, lane);
    step1<2, 2>(v, lane);
    step1<1, 1>(v, lane);
    return v;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int id) {
    return (static_cast<uint64_t>(key) << 32) | (0xffffffffu - static_cast<uint32_t>(id));
}

// The candidates slot[0..C) (composites, C <= 128) sorted descending and cut
// to 64: lane i returns the i-th largest (zero past C).
//
// With words set (a constant at every call), the network moves 32-bit words
// where that is exact.  A candidate's word is its key's distance above kb (a
// key no candidate is below) shifted left by 7, with 127 - (its slot) in the
// low bits: words order as the keys do while every distance stays below
// 2^25, and the low bits make them unique.  Equal keys come out in slot
// order, which is not id order (slots are filled lane by lane), so a sorted
// run of equal keys, or equal keys on both sides of the 64th place, sends the
// candidates through the network again as composites.  A step of the network
// moves one register instead of two and compares 32 bits instead of 64.
// C = 128 takes the composites too: its last slot's word could be zero, the
// value of an empty place.  That pays where many rows keep the VALU busy
// (1.9 % per prefill phase of 65,536 rows of 2049 blocks); a launch of few
// rows waits on the chain of steps instead, which the tie checks and the
// second LDS read lengthen as much as the narrower network shortens it.
__device__ __forceinline__ uint64_t sorted_top64(const uint64_t *slot, int C, uint32_t kb, int lane,
                                                 bool words) {
    if (words && C <= 127) {   // uniform
        const uint32_t d0 = static_cast<uint32_t>((lane < C ? slot[lane] : 0ull) >> 32) - kb;
        const uint32_t d1 = static_cast<uint32_t>((lane + 64 < C ? slot[lane + 64] : 0ull) >> 32) - kb;
        const bool far = (lane < C && d0 >= (1u << 25)) || (lane + 64 < C && d1 >= (1u << 25));
        if (ballot(far) == 0) {   // uniform
            const uint32_t w0 = lane < C ? (d0 << 7) | static_cast<uint32_t>(127 - lane) : 0u;
            const uint32_t w1 = lane + 64 < C ? (d1 << 7) | static_cast<uint32_t>(63 - lane) : 0u;
            uint32_t u, rest = 0;   // rest: the words left out of the 64 (zero if empty)
            if (C <= 64) u = sort64_desc(w0, lane);
            else u = top64_of_128(w0, w1, lane, &rest);
            const int n = C < 64 ? C : 64;
            const uint32_t next = static_cast<uint32_t>(
                __builtin_amdgcn_ds_bpermute((lane + 1) << 2, static_cast<int>(u)));
            const uint32_t last = static_cast<uint32_t>(
                __builtin_amdgcn_readlane(static_cast<int>(u), 63));
            const bool tie = (lane + 1 < n && (u >> 7) == (next >> 7)) ||
                             (rest != 0 && (rest >> 7) == (last >> 7));
            if (ballot(tie) == 0) return lane < n ? slot[127 - (u & 127)] : 0ull;
        }
    }
    // the second half is read only when there is one: a launch of few rows
    // waits on every read
    const uint64_t v0 = lane < C ? slot[lane] : 0ull;
    if (C <= 64) return sort64_desc(v0, lane);
    const uint64_t v1 = lane + 64 < C ? slot[lane + 64] : 0ull;
    return top64_of_128(v0, v1, lane);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}

// Exclusive prefix sum over the wave with DPP: shifts by 1, 2, 4, 8 within
// each row of 16 lanes (lanes without a source add 0), then row 1 and 3 add
// the last lane of the row below (row_bcast:15), rows 2 and 3 add lane 31
// (row_bcast:31).
__device__ __forceinline__ int wave_excl_scan(int x, int lane, int *total) {
    uint32_t v = static_cast<uint32_t>(x);
    v += dpp_or_zero<0x111, 0xF>(v);   // row_shr:1
    v += dpp_or_zero<0x112, 0xF>(v);   // row_shr:2
    v += dpp_or_zero<0x114, 0xF>(v);   // row_shr:4
    v += dpp_or_zero<0x118, 0xF>(v);   // row_shr:8
    v += dpp_or_zero<0x142, 0xA>(v);   // row_bcast:15 into rows 1, 3
    v += dpp_or_zero<0x143, 0xC>(v);   // row_bcast:31 into rows 2, 3
    *total = __builtin_amdgcn_readlane(static_cast<int>(v), 63);
    return static_cast<int>(v) - x;
}

// The register-held row lengths, in 64-wide columns: a row of nj columns
// takes the first case >= nj.  So the columns below the case before it are
// always full, and only the ones above can hold padding.
constexpr int kTopkCases[] = {1, 2, 4, 8, 16, 24, 32, 33, 40, 48, 64};
constexpr int full_columns(int npl) {
    int prev = 0;
    for (int c : kTopkCases) {
        if (c == npl) return prev;
        prev = c;
    }
    return 0;
}


// Padding past the row: a NaN (never >= a threshold) whose bits, read as a
// signed integer (-1), rank above every negative float and below every
// non-negative one.
constexpr uint32_t kTopkPad = 0xffffffffu;

// The row's raw fp32 bits into registers (NPL > 0): lane l gets block id
// j*64 + l in xr[j], the pad past nb.  Raw buffer loads bounded by the row
// (reads past nb return 0, no branch), then the pad substituted past nb; the
// column's byte offset is a constant added to the lane's, so it folds into
// the instruction's immediate offset (no per-column address math).
template <int NPL>
__device__ __forceinline__ void topk_row_load(const float *srow, int nb, int lane,
                                              uint32_t (&xr)[NPL > 0 ? NPL : 1]) {
    if constexpr (NPL > 0) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(srow), 0, nb * 4, 0x00020000 /* 32-bit elements, raw */);
        constexpr int kFull = full_columns(NPL);
        #pragma unroll
        for (int j = 0; j < NPL; ++j) {
            const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4 + j * 256, 0, 0);
            xr[j] = j < kFull || lane < nb - 64 * j ? x : kTopkPad;
        }
    }
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
// by bitonic networks.  Any other C takes the exact path: a 32-step
// ballot bisection for the kk-th largest key over every value, then ties in
// id order.
//
// MANY: the launch of four rows per workgroup over many rows, bound by the
// VALU's throughput; it takes the steps with fewer VALU ops even where they
// lengthen a row's chain of dependent steps (the candidate mask, the sort of
// 32-bit words).  Without it, a launch of few rows, each row's latency is
// what counts.
//
// One wave selects row srow (nb values, the raw bits already in xr when NPL
// > 0) and writes ids_row[0, k) and, when vals_row is set, vals_row[0, k).
// slot (128 composites) and stash (64*NPL words) are the wave's own LDS.
template <int NPL, bool MANY>
__device__ __forceinline__ void topk_row_select(const float *srow, int nb, int k,
                                                const uint32_t (&xr)[NPL > 0 ? NPL : 1],
                                                int32_t *ids_row, float *vals_row,
                                                uint64_t *slot, uint32_t *stash, int lane) {
    const int kk = min(k, nb);
    const int nj = (nb + 63) >> 6;               // 64-wide columns of the row
    const uint64_t lt = (1ull << lane) - 1ull;
    if constexpr (NPL > 0) {
        // the row's values, for the candidates' second look (lane l keeps its
        // own column values at [j*64 + l]: only the writing lane reads them)
        #pragma unroll
        for (int j = 0; j < NPL; ++j) stash[j * 64 + lane] = xr[j];
    }
    auto key = [&](int j) -> uint32_t {
        const int id = j * 64 + lane;
        if constexpr (NPL > 0) {
            return order_key(__builtin_bit_cast(float, xr[j]));   // pads are NaN: key 0
        } else {
            return id < nb ? order_key(srow[id]) : 0u;
        }
    };
    const int jmax = NPL > 0 ? NPL : nj;   // a constant when values are in registers

    uint64_t v = 0;
    bool done = false;
    if constexpr (NPL > 0 && NPL <= 2) {
        // At most 128 blocks: every value is already in the lane's registers,
        // so the whole row is sorted as composites, with no threshold, count
        // or compaction in front (pads past nb rank last).  Selector launches
        // in graphs, 256 rows: 64 blocks, k = 16: 2.57 -> 2.19 us; 100 blocks,
        // k = 64: 4.73 -> 2.78 us; 65,536 rows of 64 blocks: 26.2 -> 19.2 us.
        if (kk > 0) {
            const uint64_t c0 = lane < nb ? composite(key(0), lane) : 0ull;
            if constexpr (NPL == 1) {
                v = sort64_desc(c0, lane);
            } else {
                const uint64_t c1 = lane + 64 < nb ? composite(key(1), lane + 64) : 0ull;
                v = top64_of_128(c0, c1, lane);
            }
            done = true;
        }
    } else if constexpr (NPL > 0) {
        if (kk > 0) {
            // 1. samples of the fp32 bits as signed integers.  Few rows: the
            //    per-lane top two (two ops a column, a short chain).  Many
            //    rows (VALU-bound) with at least nine columns: the maxima of
            //    three column groups, about one op per three columns
            //    (v_max3_i32).  Either way kk samples >= th are kk values >=
            //    th.  On the prefill chunk's scores both give pools of about
            //    74 candidates at 2049 blocks and k = 64 (a group of 11 of
            //    2049 values reaches the 64th-largest of 192 group maxima
            //    with probability 1/3, so p = 1 - (2/3)^(1/11) ~ 3.6 %).
            constexpr bool kGroups = MANY && NPL >= 9;
            uint32_t s1, s2, s3 = 0;
            if constexpr (kGroups) {
                constexpr int G1 = NPL / 3, G2 = 2 * NPL / 3;
                int32_t g0 = INT32_MIN, g1 = INT32_MIN, g2 = INT32_MIN;
                #pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const int32_t x = static_cast<int32_t>(xr[j]);
                    if (j < G1) g0 = max(g0, x);
                    else if (j < G2) g1 = max(g1, x);
                    else g2 = max(g2, x);
                }
                s1 = static_cast<uint32_t>(g0) ^ 0x80000000u;
                s2 = static_cast<uint32_t>(g1) ^ 0x80000000u;
                s3 = static_cast<uint32_t>(g2) ^ 0x80000000u;
            } else {
                int32_t m1 = INT32_MIN, m2 = INT32_MIN;
                #pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const int32_t x = static_cast<int32_t>(xr[j]);
                    m2 = max(min(m1, x), min(max(m1, x), m2));   // median of three: v_med3_i32
                    m1 = max(m1, x);
                }
                s1 = static_cast<uint32_t>(m1) ^ 0x80000000u;
                s2 = static_cast<uint32_t>(m2) ^ 0x80000000u;
            }
            // 2. th = the kk-th largest of the samples, to 16 leading bits
            //    (bisection on the biased bits, a ballot per sample set and
            //    step): any th is correct, the low bits only tighten C
            uint32_t T = 0;
            for (int bit = 31; bit >= 16; --bit) {
                const uint32_t cand = T | (1u << bit);
                int cnt = __popcll(ballot(s1 >= cand)) + __popcll(ballot(s2 >= cand));
                if constexpr (kGroups) cnt += __popcll(ballot(s3 >= cand));
                if (cnt >= kk) T = cand;
            }
            const float th = __builtin_bit_cast(float, T ^ 0x80000000u);
            // 3. candidates x >= th as a per-lane bitmask over j.  Many rows:
            //    shifted in from the highest column down, two VALU ops a
            //    column but one chain of dependent ops; few rows, which wait
            //    on that chain: the compiler's tree of selects and ORs.
            uint32_t mlo = 0, mhi = 0;
            if constexpr (MANY) {
                #pragma unroll
                for (int j = NPL - 1; j >= 0; --j) {
                    const float x = __builtin_bit_cast(float, xr[j]);
                    if (j < 32) mlo = shift_in_ge(mlo, x, th);
                    else mhi = shift_in_ge(mhi, x, th);
                }
                // the masks' widths, which the compiler cannot see through
                // the asm: with them it sizes the compaction loop below
                if constexpr (NPL < 32) mlo &= (1u << NPL) - 1u;
                if constexpr (NPL > 32 && NPL < 64) mhi &= (1u << (NPL - 32)) - 1u;
            } else {
                #pragma unroll
                for (int j = 0; j < NPL; ++j) {
                    const bool c = __builtin_bit_cast(float, xr[j]) >= th;
                    if (j < 32) mlo |= static_cast<uint32_t>(c) << j;
                    else mhi |= static_cast<uint32_t>(c) << (j - 32);
                }
            }
            const int cnt = __popc(mlo) + __popc(mhi);
            int C = 0;
            int off = wave_excl_scan(cnt, lane, &C);
            if (C >= kk && C <= 128) {
                // 4. compact the candidates' exact composites into LDS: up to
                //    four per lane per round, their values read back from the
                //    lane's own stash
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
                    for (int r = 0; r < 4; ++r)
                        x4[r] = id4[r] >= 0 ? __builtin_bit_cast(float, stash[id4[r]]) : 0.0f;
                    #pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (id4[r] >= 0) slot[off++] = composite(order_key(x4[r]), id4[r]);
                    more = ballot((mlo | mhi) != 0);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                v = sorted_top64(slot, C, order_key(th), lane, MANY);
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
            if (sel) slot[base + __popcll(ms & lt)] = composite(kj, id);
            base += __popcll(ms);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        v = sort64_desc(lane < kk ? slot[lane] : 0ull, lane);
    }

    if (lane < k) {
        int32_t id = -1;
        float val = -__builtin_inff();
        if (lane < kk) {
            id = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(v));
            if constexpr (NPL > 0) val = __builtin_bit_cast(float, stash[id]);
            else val = srow[id];
        }
        ids_row[lane] = id;
        if (vals_row) vals_row[lane] = val;
    }
}

}  // namespace
}  // namespace qsa
