// qsa_internal.h -- launchers shared between the C-ABI layer and the kernel
// files of libqsa.so (gfx950 / CDNA4 only).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

// Blocks per MFMA scorer tile: the N extent of v_mfma_f32_32x32x16_f16 (two
// 16-block column tiles in the wide scorer's v_mfma_f32_16x16x32_f16 form).
constexpr int kTileBlocks = 32;
// Queries per wave (M = 32 rows = 16 queries x 2 heads) and waves per group.
constexpr int kWaveQueries = 16;
constexpr int kScoreWaves = 4;
constexpr int kGroupQueries = kWaveQueries * kScoreWaves;

// Logical workgroup id such that the workgroups the hardware places on one
// XCD (consecutive ids modulo 8 land on consecutive XCDs) get a contiguous
// logical range.  Bijective for any grid size.  The scorers order their work
// by it so that neighbouring work shares an XCD's L2, and the selectors order
// their rows by it so that a row is selected on the XCD that scored it: with
// few rows the scores are still in that L2 when the selector reads them.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t bid, uint32_t nblk) {
    const uint32_t q = nblk / 8, r = nblk % 8;
    const uint32_t x = bid % 8, idx = bid / 8;
    return x * q + (x < r ? x : r) + idx;
}

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

// Two fp32 values to packed fp16 bits by v_cvt_pk_f16_f32: round to nearest
// even by the MODE register, fp16 subnormals kept, overflow to infinity, and
// a NaN becomes the quiet NaN with the input's sign and top 10 fraction bits,
// i.e. f16_rne on both halves.  The vector conversion kernel is built from
// this instruction, and its test compares all 2^32 fp32 patterns with the
// oracle's rounding, so the scorers that convert on load with it inherit that
// check.
typedef _Float16 qsa_half2 __attribute__((ext_vector_type(2)));
typedef float qsa_float2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(qsa_float2{a, b}, qsa_half2));
}

// Eight fp32 values to fp16 bits, as four packed conversions.
__device__ __forceinline__ uint4 f16x8(const float4 &x0, const float4 &x1) {
    return make_uint4(f16x2(x0.x, x0.y), f16x2(x0.z, x0.w), f16x2(x1.x, x1.y), f16x2(x1.z, x1.w));
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
    // Added to the partial last block's score after its head sum (fp32):
    // 1e9 under the forced-tail rule, else 0 (then nothing is added).
    float tail_add;
};

// Full-block MFMA scorer over blocks [0, nf).  Many query rows: one kernel
// per head pass of up to eight heads; few: the small scorer.  With tail
// (requires nf > 0) block nf is scored too, in the fixed order of the tail
// model, inside the same launches.  With q32 set (src32_ok) the queries are
// read as fp32 in the layout of g.q16, converted on load (f16_rne bits), and
// their fp16 bits written to q16w when it is set: the G*H*D elements of every
// token row, nothing between rows.
// Where a scorer that also selects (the fused form) writes the top-k of
// score row g*nq + t: ids[(g*dst_group_rows + dst_row0 + t)*ld_ids + j],
// j < k, and vals likewise when set.
struct FusedSelect {
    int32_t *ids;
    int64_t ld_ids;
    float *vals;
    int32_t k;
    int64_t dst_group_rows, dst_row0;
    // streaming form: the running selection of qsa_stream_row.h, no score
    // written (shapes with one workgroup per query group over all blocks,
    // one head pass, at most 65536 blocks)
    bool stream;
    // the scores written, then selected at the end of the same launch
    bool fused;
};

// Whether the streaming selection serves this shape (the decode, small and
// split-block shapes and more than 8 heads take the two-launch path).
bool stream_select_serves(const ScoreGeom &g, bool tail);

// With fs set, shapes the fused form serves (one workgroup per query group
// over all blocks, one head pass, 513-1024 or 2049-2112 blocks) are scored
// and selected in the one launch, and *selected is set; otherwise the
// selection is left to the caller.
hipError_t launch_score_full(const ScoreGeom &g, bool tail, hipStream_t s,
                             const float *q32 = nullptr, uint16_t *q16w = nullptr,
                             const FusedSelect *fs = nullptr, bool *selected = nullptr);

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

// Decode steps: at most one MFMA row block of queries per KV head (nq <=
// 16 / head pairs) and at least one full block.  The decode scorer of
// qsa_decode.hip: one wave per 32-block tile, operands straight from memory,
// the same bits as the small scorer; with tail the partial block nf too.
bool decode_rows(const ScoreGeom &g);
hipError_t launch_score_decode(const ScoreGeom &g, bool tail, hipStream_t s,
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

// Block keys: kblk[g][b] = the fp16-rounded mean of the tokens of block b of
// KV head g (qsa_blockkeys.hip).  D in {64, 128}, 1 <= bs <= 8192.
hipError_t launch_block_keys(const uint16_t *k_tok, int64_t tok_stride, uint16_t *kblk,
                             int64_t khs, int32_t G, int32_t D, int64_t n_kv, int32_t bs,
                             hipStream_t s);

// Attention of every query head over the tokens of its row's selected
// blocks (qsa_attention.hip).  D in {64, 128}, H in [1, 16].
// With ws (ws_floats floats), few rows are split over several workgroups
// whose partial results a second launch merges.
hipError_t launch_attention(const uint16_t *q16, int64_t qts, const uint16_t *k_tok,
                            const uint16_t *v_tok, int64_t kvts, const int32_t *ids, int64_t ld_ids,
                            float *out, int64_t ots, int32_t G, int32_t nq, int32_t H, int32_t D,
                            int64_t n_kv, int32_t bs, int32_t k, float *ws, int64_t ws_floats,
                            hipStream_t s);

// Workgroups per row the attention uses when a workspace allows.
int64_t attention_splits(int64_t rows, int32_t bs, int32_t k);

// rows of row_len elements at a stride of stride elements (both arrays)
hipError_t launch_convert_rows(const float *src, uint16_t *dst, int64_t rows, int64_t row_len,
                               int64_t stride, hipStream_t s);

}  // namespace qsa
