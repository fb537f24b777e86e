// qsa_stream_row.h -- the running per-row selection of the streaming scorer
// (qsa_score.hip, QSA_STREAM_SELECT): each wave keeps, for each of its score
// rows, a buffer of candidate blocks in LDS while the block tiles stream by,
// so that the top-k of the row ("selection/topk", Strata pull request #228,
// part 1) is found without a score matrix in memory.
//
// A row's buffer holds (score bits, block id) pairs in block-id order: tiles
// arrive in block order, each tile's candidates are appended in lane (block)
// order, and every compaction below keeps the survivors' relative order.  So
// a tie of scores is always resolved by buffer position, which is the
// selector's tie rule (lower id first), and the final sort can use positions
// in place of ids.
//
// Admission: a block enters its row's buffer when its order key is at least
// the row's admission key adm (NaN always enters; its key is the lowest).
// When the buffer is full the row is compacted: a ballot bisection over the
// top 16 bits of the order keys finds T, the largest 16-bit-prefix key with
// at least kk entries >= T; entries below T are dropped (kk better ones are
// kept) and adm becomes T.  If that frees too little (many equal scores) or T
// is 0 (fewer than kk numbers), the bisection runs on to the exact kk-th key
// and exactly kk entries are kept: those with larger keys, then the ties in
// buffer (id) order; adm becomes T + 1, since a later block, having a larger
// id, needs a strictly larger key.  Either way every block of the row's true
// top-kk is admitted and never dropped: anything refused or dropped had kk
// entries ranked above it.
#pragma once

#include "qsa_topk_row.h"

namespace qsa {
namespace {

// Candidates per row buffer: two per lane for the compaction and final sort.
constexpr int kStreamCap = 128;

// Orders this wave's LDS accesses of other lanes' data (a write of one lane
// before a read of another) without a workgroup barrier.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The wave's mask of lanes where p holds.  The bool form of the builtin: the
// int form (__ballot) goes through a select and a compare per call.
__device__ __forceinline__ uint64_t ballot_b(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// x, known to be the same in every lane, as a scalar-register value.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// v with lane r's element replaced by x (r uniform).
__device__ __forceinline__ uint32_t lane_set(uint32_t v, int lane, int r, uint32_t x) {
    return lane == r ? x : v;
}

// The float threshold th such that !(x < th) admits every score x >= +0 with
// order key >= adm (and every NaN): -inf when adm is at or below the key of
// +0, else the smallest non-negative float of that key, capped at +inf (the
// cap only widens the admission).  Scores are sums of relu outputs, never
// negative, so keys below that of +0 do not occur.
__device__ __forceinline__ float stream_admit_floor(uint32_t adm) {
    if (adm <= 0x80000000u) return -__builtin_inff();
    const uint32_t b = adm - 0x80000000u;
    return __builtin_bit_cast(float, b < 0x7f800000u ? b : 0x7f800000u);
}

// Compacts one row buffer (vb scores, ib block ids; c > 0 entries, c >= kk)
// as described above.  Returns the number kept (>= kk, <= kStreamCap -
// kTileBlocks, so that a tile's candidates always fit after it); *adm gets
// the row's new admission key and *kb a key no kept or later-admitted
// number is below.
__device__ __forceinline__ int stream_compact(uint32_t *vb, uint16_t *ib, int c, int kk, int lane,
                                              uint32_t *adm, uint32_t *kb) {
    wave_lds_sync();
    const uint32_t v0 = vb[lane], v1 = vb[64 + lane];
    const uint32_t i0 = ib[lane], i1 = ib[64 + lane];
    const bool ok0 = lane < c, ok1 = lane + 64 < c;
    const uint32_t k0 = ok0 ? order_key(__builtin_bit_cast(float, v0)) : 0u;
    const uint32_t k1 = ok1 ? order_key(__builtin_bit_cast(float, v1)) : 0u;
    auto count_ge = [&](uint32_t t) {
        return __popcll(ballot_b(k0 >= t)) + __popcll(ballot_b(k1 >= t));
    };
    uint32_t T = 0;
    for (int bit = 31; bit >= 16; --bit) {
        const uint32_t cand = T | (1u << bit);
        if (count_ge(cand) >= kk) T = cand;
    }
    bool keep0 = ok0 && k0 >= T, keep1 = ok1 && k1 >= T;
    int kept = __popcll(ballot_b(keep0)) + __popcll(ballot_b(keep1));
    uint32_t a = T;
    const uint64_t lt = (1ull << lane) - 1ull;
    if (T == 0 || kept > kStreamCap - kTileBlocks) {   // uniform
        for (int bit = 15; bit >= 0; --bit) {
            const uint32_t cand = T | (1u << bit);
            if (count_ge(cand) >= kk) T = cand;
        }
        const bool gt0 = ok0 && k0 > T, gt1 = ok1 && k1 > T;
        const int need = kk - (__popcll(ballot_b(gt0)) + __popcll(ballot_b(gt1)));
        const bool eq0 = ok0 && k0 == T, eq1 = ok1 && k1 == T;
        const uint64_t me0 = ballot_b(eq0), me1 = ballot_b(eq1);
        keep0 = gt0 || (eq0 && __popcll(me0 & lt) < need);
        keep1 = gt1 || (eq1 && __popcll(me0) + __popcll(me1 & lt) < need);
        kept = kk;
        a = T + 1;
    }
    const uint64_t mk0 = ballot_b(keep0), mk1 = ballot_b(keep1);
    const int p0 = __popcll(mk0 & lt);
    const int p1 = __popcll(mk0) + __popcll(mk1 & lt);
    // every entry is in registers: the moves (always to a lower or equal
    // position) cannot overwrite one not yet read
    wave_lds_sync();
    if (keep0) {
        vb[p0] = v0;
        ib[p0] = static_cast<uint16_t>(i0);
    }
    if (keep1) {
        vb[p1] = v1;
        ib[p1] = static_cast<uint16_t>(i1);
    }
    *adm = a;
    *kb = T;
    return kept;
}

// The row's selection from its buffer (c <= kStreamCap entries, c >= kk):
// the first kk entries by (key desc, position asc), sorted; ids_row[0, k)
// and vals_row[0, k) (when set) written as the selector writes them.  slot
// is this wave's 128-entry composite area in LDS.
__device__ __forceinline__ void stream_final(const uint32_t *vb, const uint16_t *ib, int c, int k,
                                             int kk, uint32_t kb, uint64_t *slot, int32_t *ids_row,
                                             float *vals_row, int lane) {
    wave_lds_sync();
    const uint32_t v0 = vb[lane], v1 = vb[64 + lane];
    if (lane < c) slot[lane] = composite(order_key(__builtin_bit_cast(float, v0)), lane);
    if (lane + 64 < c) slot[64 + lane] = composite(order_key(__builtin_bit_cast(float, v1)), 64 + lane);
    wave_lds_sync();
    const uint64_t v = sorted_top64(slot, c, kb, lane, true);
    if (lane < k) {
        int32_t id = -1;
        float val = -__builtin_inff();
        if (lane < kk) {
            const int pos = static_cast<int>(0xffffffffu - static_cast<uint32_t>(v));
            id = ib[pos];
            val = __builtin_bit_cast(float, vb[pos]);
        }
        ids_row[lane] = id;
        if (vals_row) vals_row[lane] = val;
    }
    wave_lds_sync();   // the slots are reused by the next row
}

}  // namespace
}  // namespace qsa
