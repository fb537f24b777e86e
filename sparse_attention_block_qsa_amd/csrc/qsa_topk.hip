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

// R / rows_per_group for a wave-uniform row R: a 32-bit division (a few
// scalar ops) when the rows fit in 31 bits, else the 64-bit one (about 190).
__device__ __forceinline__ int64_t row_group(int64_t R, int64_t rows_per_group, int64_t total_rows) {
    if (total_rows <= 0x7fffffff)   // uniform
        return static_cast<uint32_t>(R) / static_cast<uint32_t>(rows_per_group);
    return R / rows_per_group;
}

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
template <int NPL, bool MANY>
__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
    __shared__ uint64_t slot[4][128];   // one per wave of the workgroup (at most four)
    // the row's values, for the candidates' second look (lane l keeps its own
    // column values at [j*64 + l]: only the writing lane reads them back)
    __shared__ uint32_t stash[NPL > 0 ? 4 : 1][NPL > 0 ? 64 * NPL : 1];
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
        // Raw buffer loads bounded by the row (reads past nb return 0, no
        // branch), then the pad substituted past nb.
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(srow), 0, nb * 4, 0x00020000 /* 32-bit elements, raw */);
        constexpr int kFull = full_columns(NPL);
        #pragma unroll
        for (int j = 0; j < NPL; ++j) {
            // the column's byte offset is a constant added to the lane's: it
            // folds into the instruction's immediate offset (no per-column
            // address math on the VALU)
            const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4 + j * 256, 0, 0);
            xr[j] = j < kFull || lane < nb - 64 * j ? x : kPad;
        }
        #pragma unroll
        for (int j = 0; j < NPL; ++j) stash[w][j * 64 + lane] = xr[j];
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
    if constexpr (NPL > 0) {
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
                        x4[r] = id4[r] >= 0 ? __builtin_bit_cast(float, stash[w][id4[r]]) : 0.0f;
                    #pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (id4[r] >= 0) slot[w][off++] = composite(order_key(x4[r]), id4[r]);
                    more = ballot((mlo | mhi) != 0);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                v = sorted_top64(slot[w], C, order_key(th), lane, MANY);
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
        v = sort64_desc(lane < kk ? slot[w][lane] : 0ull, lane);
    }

    if (lane < a.k) {
        int32_t id = -1;
        float val = -__builtin_inff();
        if (lane < kk) {
            id = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(v));
            if constexpr (NPL > 0) val = __builtin_bit_cast(float, stash[w][id]);
            else val = srow[id];
        }
        a.ids[drow * a.ld_ids + lane] = id;
        if (a.vals) a.vals[drow * a.ld_ids + lane] = val;
    }
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
