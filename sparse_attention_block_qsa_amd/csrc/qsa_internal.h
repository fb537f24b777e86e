// qsa_internal.h -- launchers shared between the C-ABI layer and the kernel
// files of libqsa.so (gfx950 / CDNA4 only).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Blocks per MFMA scorer tile: the N extent of v_mfma_f32_32x32x16_f16.
constexpr int kTileBlocks = 32;
// Queries per wave (M = 32 rows = 16 queries x 2 heads) and waves per group.
constexpr int kWaveQueries = 16;
constexpr int kScoreWaves = 4;
constexpr int kGroupQueries = kWaveQueries * kScoreWaves;

// fp32 -> fp16 bits, round to nearest even.  v_cvt_f16_f32 rounds by the
// MODE register, which is round-to-nearest-even for compute kernels, keeps
// fp16 subnormals and overflows to infinity.  NaN is rewritten explicitly so
// its bits are defined: quiet, with the sign and the top 10 fraction bits of
// the input.
__device__ __forceinline__ uint32_t f16_rne(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    uint32_t h = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
    if ((u & 0x7fffffffu) > 0x7f800000u)
        h = ((u >> 16) & 0x8000u) | 0x7e00u | ((u >> 13) & 0x3ffu);
    return h;
}

// Eight fp32 values to fp16 bits (two dwords each), f16_rne per element.
__device__ __forceinline__ uint4 f16x8_exact(const float4 &x0, const float4 &x1) {
    return make_uint4(f16_rne(x0.x) | (f16_rne(x0.y) << 16), f16_rne(x0.z) | (f16_rne(x0.w) << 16),
                      f16_rne(x1.x) | (f16_rne(x1.y) << 16), f16_rne(x1.z) | (f16_rne(x1.w) << 16));
}

// The same with the bare hardware conversion: equal to f16x8_exact for every
// input that is not a NaN (max_mag_bits tells whether there is one).
__device__ __forceinline__ uint4 f16x8_cvt(const float4 &x0, const float4 &x1) {
    auto h = [](float x) -> uint32_t { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)); };
    return make_uint4(h(x0.x) | (h(x0.y) << 16), h(x0.z) | (h(x0.w) << 16),
                      h(x1.x) | (h(x1.y) << 16), h(x1.z) | (h(x1.w) << 16));
}

// Largest magnitude bit pattern of eight fp32 values: a NaN among them iff
// the result is > 0x7f800000.
__device__ __forceinline__ uint32_t max_mag_bits(const float4 &x0, const float4 &x1) {
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t m = 0;
    #pragma unroll
    for (int e = 0; e < 8; ++e) m = max(m, __builtin_bit_cast(uint32_t, xs[e]) & 0x7fffffffu);
    return m;
}

struct ScoreGeom {
    const uint16_t *q16;
    int64_t qts;          // elements between tokens
    const uint16_t *kblk;
    int64_t khs;          // elements between KV heads
    float *scores;
    int64_t ld_s;
    int32_t G, nq, H, D;
    int64_t nf;           // full blocks
};

// Full-block MFMA scorer over blocks [0, nf).  Many query rows: one kernel
// per head pass of up to eight heads; few: the small scorer.  With tail
// (requires nf > 0) block nf is scored too, in the fixed order of the tail
// model, inside the same launches.  With q32 set (src32_ok) the queries are
// read as fp32 in the layout of g.q16, converted on load (f16_rne bits), and
// their fp16 bits written to q16w when it is set: the G*H*D elements of every
// token row, nothing between rows.
hipError_t launch_score_full(const ScoreGeom &g, bool tail, hipStream_t s,
                             const float *q32 = nullptr, uint16_t *q16w = nullptr);

// Few query rows (fewer than 256 groups of 64 over the KV heads): the
// scorer of qsa_small.hip, latency-bound shapes.
bool small_rows(const ScoreGeom &g);

// fp32 queries the scorers can read directly (16-byte vector loads).
bool src32_ok(const float *q32, int64_t qts);

// The small scorer: blocks [0, nf) and, with tail, the partial block nf in
// the fixed order of the tail model (also when nf == 0).  With q32 set the
// queries are read as fp32 (layout of g.q16), converted on load, and their
// fp16 bits written to q16w: the G*H*D elements of every token row, nothing
// between rows.
hipError_t launch_score_small(const ScoreGeom &g, bool tail, hipStream_t s,
                              const float *q32 = nullptr, uint16_t *q16w = nullptr);

// Fixed-order scorer of the single block b_tail, standalone (used when there
// is no full block to share the query reads with).
hipError_t launch_tail(const ScoreGeom &g, int64_t b_tail, hipStream_t s);

struct TopkGeom {
    const float *scores;
    int64_t ld_s;
    int32_t *ids;
    int64_t ld_ids;
    float *vals;
    // row (grp, t), t < rows_per_group:
    //   source row      grp * src_group_rows + t
    //   destination row grp * dst_group_rows + dst_row0 + t
    int64_t n_groups, rows_per_group, src_group_rows, dst_group_rows, dst_row0;
    int32_t nb, k;
};

hipError_t launch_topk(const TopkGeom &g, hipStream_t s);

hipError_t launch_convert(const float *src, uint16_t *dst, int64_t n, hipStream_t s);

// rows of row_len elements at a stride of stride elements (both arrays)
hipError_t launch_convert_rows(const float *src, uint16_t *dst, int64_t rows, int64_t row_len,
                               int64_t stride, hipStream_t s);

}  // namespace qsa
