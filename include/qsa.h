/*
 * qsa.h -- C ABI of libqsa.so, the MI355X (gfx950) QSA block-score select
 * phase.
 *
 * The phase (Strata pull request #228, part 1 "qsa_block_scores_wmma: the
 * prompt scorer arm on tensor cores": the score formula in the first
 * paragraph, and the paragraph after the bench table, which lists the
 * phase as scores + selection/top-k + the fp16 conversion + the batch loop):
 *
 *   1. convert the fp32 query activations to fp16 (round to nearest even);
 *   2. for every KV head g, query t and KV block b
 *        score(g, t, b) = sum_{h < H} relu( sum_{i < D} k[g, b, i] * q[t, g, h, i] )
 *      with fp16 operands and fp32 accumulation; the last, partial block
 *      (when n_kv is not a multiple of the block size) by a separate
 *      fixed-order kernel;
 *   3. per (g, t) row keep the top-k blocks, by score descending with ties
 *      to the lower block id.
 *
 * Every score lies within the page's arithmetic contract
 *   B = 2^-9.5 * S + 8 * 2^-24 * |score_ref|,  S = sum_h sum_i |k[i] * q_h[i]|
 * of the float64 value (same page, "arithmetic contract" paragraph).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers (memory the caller allocated on the GPU
 *    that owns `stream`).  fp16 data is passed as its raw bits (uint16_t).
 *  - Strides are in ELEMENTS of the pointed-to type.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; nothing is synchronised or allocated,
 *    and nothing is kept between calls except the fixed per-GPU scratch
 *    array of qsa_select_phase_noalloc.  Calls are thread-safe (calls of
 *    qsa_select_phase_noalloc that overlap on one GPU race on its array).
 *  - Refusal is clean: when a call returns anything but QSA_OK, nothing was
 *    launched and no output byte was written.  Errors that happen on the
 *    device after a successful launch surface at the caller's next
 *    synchronisation of the stream.
 *  - Write sets are exact: an entry point writes the output cells documented
 *    for it and nothing else (pad columns and memory around the outputs are
 *    left untouched).
 *  - Inputs must be finite; non-finite inputs give unspecified scores (the
 *    call still completes).
 *
 * Layouts
 *  q16[t * q_tok_stride + (g*H + h) * D + i]      token-major queries, the same as
 *                                                 a GQA query tensor [tokens][G*H][D]
 *  kblk[g * kblk_head_stride + b * D + i]         one key vector per KV block
 *  scores[(g*nq + t) * ld_s + b]                  fp32, row r = g*nq + t
 *  ids[(g*nq + t) * ld_ids + j], vals[...]        j < k
 */
#ifndef QSA_H
#define QSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qsa_status {
    QSA_OK = 0,
    QSA_ERR_ARG = 1,         /* NULL where data is needed, negative size, stride
                                or leading dimension too small, size overflow */
    QSA_ERR_UNSUPPORTED = 2, /* geometry outside the supported set: D not in
                                {64, 128}, H outside [1, 16], k > 64, block size
                                < 1, a pointer or stride not 16-byte aligned
                                where the kernels load 16-byte vectors */
    QSA_ERR_HIP = 3,         /* the HIP runtime refused a launch */
    QSA_ERR_TOO_LARGE = 4    /* qsa_select_phase_noalloc: the work does not fit
                                the library's fixed scratch array */
} qsa_status;

#define QSA_ABI_VERSION 7
#define QSA_MAX_K 64
/* Largest block size qsa_block_keys takes (its sums stay exact in float64). */
#define QSA_BLOCK_KEYS_MAX_BS 8192
/* Size of the per-GPU device array qsa_select_phase_noalloc keeps its score
 * workspace in (64 MiB). */
#define QSA_NOALLOC_SCRATCH_BYTES (64ll << 20)

/* Version of this ABI (QSA_ABI_VERSION of the header the library was built
 * with). */
int qsa_abi_version(void);

/* Static description of a status code; never NULL. */
const char *qsa_status_string(qsa_status s);

/*
 * qsa_convert_f32_f16 -- step 1 of the phase ("the fp16 conversion",
 * Strata pull request #228, part 1, paragraph after the bench table).
 * dst[i] = fp16 bits of src[i] rounded to nearest, ties to even, for
 * 0 <= i < n.  |x| >= 65520 becomes +-inf; fp16 subnormals are produced;
 * NaN stays NaN (quiet, sign and top fraction bits kept).
 *   src  device, n floats;     dst  device, n uint16 (fp16 bits).
 * n == 0 is a no-op (pointers may then be NULL).  src and dst must not
 * overlap.  Errors: QSA_ERR_ARG (n < 0, NULL with n > 0).
 */
qsa_status qsa_convert_f32_f16(const float *src, uint16_t *dst, int64_t n, void *stream);

/* The forced-tail rule of the scorer (Strata pull request #856, "What": the
 * tail block keeps the +1e9 rule of the shared tail kernel).  Reading taken:
 * the partial last block's score, once its head sum is done, gets 1e9 added
 * in single precision, s = fl32(s + 1e9f), so that the block holding the
 * newest tokens ranks first in every row's selection whatever its keys
 * score.  It applies only when that block exists (n_kv % bs != 0). */
#define QSA_FORCE_TAIL 1u

/* Largest token stride (elements) of qsa_sparse_attention's K and V caches:
 * 64 rows of it are addressed with 32-bit byte offsets. */
#define QSA_ATTENTION_MAX_KV_STRIDE (16ll << 20)

/* qsa_select_phase / qsa_select_phase_noalloc: select inside the scorer's
 * launch where the fused scorer serves the shape (many query rows, so that
 * each workgroup scores every block of its 64 queries; H <= 8; 513-1024 or
 * 2049-2112 blocks); other shapes take the separate selector launch.  The
 * ids, values and scores are the same bits either way: the fused scorer
 * writes the scores, then each wave selects its own rows with the
 * selector's row code.  Not accepted by qsa_block_scores. */
#define QSA_FUSED_SELECT 2u

/* qsa_select_phase / qsa_select_phase_noalloc: the selection streams with the
 * scoring, and no score is written (the scope of the pages' phase, Strata
 * pull request #228, part 1: scores, then the per-query top-k; the scores
 * themselves are only the selection's input).  Where the wide scorer serves
 * the shape with one workgroup per 64 queries over all blocks (many query
 * rows, H <= 8, at most 65536 blocks), each wave keeps a running candidate
 * set per score row in LDS while the block tiles stream by, and selects from
 * it at the end of the launch: the ids and values are those of the separate
 * selector over the same scores, bit for bit, and scores_ws is not touched.
 * Other shapes take the two-launch path (scores written, then selected).
 * Takes precedence over QSA_FUSED_SELECT where it serves the shape.  Not
 * accepted by qsa_block_scores. */
#define QSA_STREAM_SELECT 4u

/*
 * qsa_block_scores -- step 2 of the phase: the score of every (g, t, b)
 * cell, b < nb = ceil(n_kv / bs).  Blocks b < nf = floor(n_kv / bs) go to the
 * MFMA full-block scorer; the partial block b = nf (present when n_kv % bs
 * != 0) is scored in a fixed order (per head a single-precision fused
 * multiply-add chain over i ascending, relu, then the head sum over h
 * ascending) that reproduces the same results bit for bit on every run
 * (Strata pull request #228, part 1, the paragraph naming the tail kernel;
 * Strata pull request #856, "What"): inside the full-block scorer's launch,
 * or by a tail kernel of its own when there is no full block.
 *   q16        device fp16 bits, layout above; q_tok_stride >= G*H*D,
 *              q16 and q_tok_stride 16-byte aligned (q_tok_stride % 8 == 0)
 *   kblk       device fp16 bits [G][>= nb][D] at kblk_head_stride >= nb*D
 *              (16-byte aligned, kblk_head_stride % 8 == 0)
 *   scores     device fp32 [G*nq][ld_s], ld_s >= nb; written: [r][0, nb)
 *   G, nq >= 0; H in [1, 16]; D in {64, 128}; n_kv >= 0; bs >= 1
 *   flags      0, or QSA_FORCE_TAIL; any other bit: QSA_ERR_ARG
 * n_kv == 0 (nb == 0), nq == 0 or G == 0: QSA_OK, nothing written.
 */
qsa_status qsa_block_scores(const uint16_t *q16, int64_t q_tok_stride,
                            const uint16_t *kblk, int64_t kblk_head_stride,
                            float *scores, int64_t ld_s,
                            int32_t G, int32_t nq, int32_t H, int32_t D,
                            int64_t n_kv, int32_t bs, uint32_t flags, void *stream);

/*
 * qsa_select_topk -- step 3 of the phase ("selection/topk", Strata pull
 * request #228, part 1; ids compared across arms in Strata pull request
 * #856).  For each row r < rows: the first min(k, nb) block ids in the order
 * (score descending, block id ascending), where scores compare numerically
 * (-0 == +0) and NaN ranks below every number; slots [min(k, nb), k) get -1.
 *   scores  device fp32 [rows][ld_s], ld_s >= nb (only [r][0, nb) is read)
 *   ids     device int32 [rows][ld_ids], ld_ids >= k; written: [r][0, k)
 *   vals    device fp32 [rows][ld_ids] or NULL; written: [r][0, k): the
 *           selected scores (bit copies), -inf in padded slots
 *   rows >= 0, nb >= 0, 0 <= k <= 64
 * k == 0 or rows == 0: QSA_OK, nothing written.  nb == 0: every slot -1.
 */
qsa_status qsa_select_topk(const float *scores, int64_t ld_s, int64_t rows, int32_t nb,
                           int32_t k, int32_t *ids, int64_t ld_ids, float *vals,
                           void *stream);

/*
 * qsa_block_keys -- the block keys the scorer reads, built from token keys:
 * the step before the phase.  The pages index one key vector k_b per KV
 * block (Strata pull request #228, part 1, score formula) but do not say how
 * it is built; the reading taken is the mean of the block's token keys:
 *   kblk[g][b][i] = fp16 nearest (ties to even) to
 *                   (1/len_b) * sum_{t in block b} k_tok[t][g][i]
 * with block b = tokens [b*bs, min((b+1)*bs, n_kv)) and len_b its length
 * (the partial last block averages its own tokens).  The mean is exact
 * before its one rounding, so the result does not depend on any summation
 * order.
 *   k_tok      device fp16 bits, token-major like a KV cache: element
 *              (t, g, i) at k_tok[t * tok_stride + g * D + i];
 *              tok_stride >= G*D; 16-byte aligned, tok_stride % 8 == 0;
 *              values must be finite
 *   kblk       device fp16 bits [G][>= nb][D] at kblk_head_stride >= nb*D
 *              (16-byte aligned, kblk_head_stride % 8 == 0);
 *              written: [g][0, nb)[0, D)
 *   G >= 0, D in {64, 128}, n_kv >= 0, 1 <= bs <= QSA_BLOCK_KEYS_MAX_BS
 * G == 0 or n_kv == 0: QSA_OK, nothing written.
 */
qsa_status qsa_block_keys(const uint16_t *k_tok, int64_t tok_stride, uint16_t *kblk,
                          int64_t kblk_head_stride, int32_t G, int32_t D, int64_t n_kv,
                          int32_t bs, void *stream);

/*
 * qsa_sparse_attention -- attention over the selected blocks: the step after
 * the phase.  The pages stop at the selection (Strata pull request #228,
 * part 1: the phase keeps each query's top-k blocks); the reading taken for
 * the step that consumes it is plain softmax attention of every query head
 * over the tokens of the blocks its (KV head, query) row selected:
 *   s_j = scale * sum_i q[t][g][h][i] * k[j][g][i],   scale = fp32(1/sqrt(D))
 *   out[t][g][h][:] = sum_j exp(s_j - max_j s_j) v[j][g][:] / sum_j exp(s_j - max_j s_j)
 * over every token j of every block b = ids[g*nq + t][slot], slot < k,
 * tokens [b*bs, min((b+1)*bs, n_kv)); ids outside [0, nb) are empty slots;
 * a row with no token gives 0.  fp16 inputs, fp32 arithmetic and output.
 * ids must not repeat a block within a row (each listed block counts once
 * per listing).
 *   q16        device fp16 bits, layout of qsa_block_scores' q16 (2-byte aligned)
 *   k_tok, v_tok  device fp16 bits, token-major: element (j, g, i) at
 *              [j * kv_tok_stride + g * D + i]; kv_tok_stride >= G*D,
 *              16-byte aligned, kv_tok_stride % 8 == 0, kv_tok_stride <=
 *              QSA_ATTENTION_MAX_KV_STRIDE (unused when n_kv == 0)
 *   ids        device int32 [G*nq][ld_ids], ld_ids >= k (the selector's ids)
 *   out        device fp32, element (t, g, h, i) at
 *              [t * out_tok_stride + (g*H + h) * D + i], out_tok_stride >= G*H*D;
 *              written: exactly those G*H*D elements of each of the nq rows
 *   ws         device fp32 workspace of ws_floats floats, or NULL.  With
 *              few rows (a decode step) each row is split over several
 *              workgroups whose partial results a second launch merges, if
 *              ws holds qsa_sparse_attention_ws_floats() floats (a smaller ws
 *              splits less; NULL: one workgroup per row).  Contents on
 *              return are unspecified; must not overlap the other buffers.
 *   G, nq >= 0; H in [1, 16]; D in {64, 128}; n_kv >= 0; bs >= 1; 0 <= k <= 64
 * nq == 0 or G == 0: QSA_OK, nothing written.  The results do not depend on
 * ws beyond fp32 rounding (the order of the partial sums).
 */
qsa_status qsa_sparse_attention(const uint16_t *q16, int64_t q_tok_stride, const uint16_t *k_tok,
                                const uint16_t *v_tok, int64_t kv_tok_stride, const int32_t *ids,
                                int64_t ld_ids, float *out, int64_t out_tok_stride, int32_t G,
                                int32_t nq, int32_t H, int32_t D, int64_t n_kv, int32_t bs,
                                int32_t k, float *ws, int64_t ws_floats, void *stream);

/* Floats of workspace qsa_sparse_attention splits its rows with for this
 * geometry (0: it would not split them). */
int64_t qsa_sparse_attention_ws_floats(int32_t G, int32_t nq, int32_t H, int32_t D, int32_t bs,
                                       int32_t k);

/*
 * qsa_select_phase -- the whole phase on one stream: convert (when q32 is
 * given), score (full blocks + tail), select.  The batch loop is folded into
 * the launch grids; with q_chunk > 0 the host walks the queries in chunks of
 * q_chunk so that the score workspace holds only G*q_chunk rows.
 *   q32       device fp32 queries (layout of q16, same q_tok_stride), 4-byte
 *             aligned, or NULL
 *   q16       device fp16 bits: the input when q32 == NULL (required then);
 *             with q32 either NULL or a buffer that receives the converted
 *             queries: exactly the G*H*D elements of each of the nq token
 *             rows are written (elements between rows, when q_tok_stride >
 *             G*H*D, are not touched).  With q32 and 16-byte aligned fp32 rows
 *             (q32 16-byte aligned, q_tok_stride % 8 == 0) the scorers convert
 *             the queries as they load them, so the conversion costs no HBM
 *             round trip of its own; storing them into q16 adds one write of
 *             the fp16 rows.  q16 == NULL with fp32 rows that are only 4-byte
 *             aligned: QSA_ERR_UNSUPPORTED (the conversion kernel would need
 *             the buffer).
 *   scores_ws device fp32 [G*qc][ld_s] workspace, qc = q_chunk > 0 ?
 *             min(q_chunk, nq) : nq; for the chunk of n <= qc queries starting
 *             at query t0, row g*n + t' holds the scores of query t0 + t'
 *             (after the call: those of the last chunk), except where
 *             QSA_STREAM_SELECT served the shape (then it is not written)
 *   ids, vals as qsa_select_topk with rows = G*nq (vals may be NULL)
 *   flags     QSA_FORCE_TAIL (as qsa_block_scores), QSA_FUSED_SELECT,
 *             QSA_STREAM_SELECT (any combination), or 0
 *   other arguments as qsa_block_scores / qsa_select_topk.
 * Workspaces must not overlap the inputs or outputs.  Errors as the three
 * stage entry points; the whole call is validated before the first launch.
 */
qsa_status qsa_select_phase(const float *q32, uint16_t *q16, int64_t q_tok_stride,
                            const uint16_t *kblk, int64_t kblk_head_stride,
                            float *scores_ws, int64_t ld_s,
                            int32_t *ids, int64_t ld_ids, float *vals,
                            int32_t G, int32_t nq, int32_t H, int32_t D,
                            int64_t n_kv, int32_t bs, int32_t k, int64_t q_chunk,
                            uint32_t flags, void *stream);

/*
 * qsa_select_phase_noalloc -- qsa_select_phase for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes the same inputs and outputs
 * (q32, q16, q_tok_stride, kblk, kblk_head_stride, ids, ld_ids, vals, flags
 * and the geometry, as qsa_select_phase) but no score workspace: the scores live in a
 * device array of QSA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from the first call on that GPU until the process ends.
 * Nothing else is allocated (no hipMalloc, hipFree or allocating library
 * call).  The GPU is the current device, which must own `stream`.
 *   q_chunk  queries per pass; 0 = as many as fit the array, i.e. the queries
 *            are walked in chunks of floor(QSA_NOALLOC_SCRATCH_BYTES /
 *            (4 * G * ld)) with ld = ceil(max(nb, 1) / 32) * 32 floats
 *            (one pass when they all fit)
 * Results are those of qsa_select_phase with the same q_chunk, bit for bit.
 * Errors: as qsa_select_phase; QSA_ERR_TOO_LARGE (nothing launched) when one
 * query's G score rows, or the q_chunk asked for, exceed the array.  With
 * QSA_STREAM_SELECT, a shape the streaming selection serves whole (q_chunk 0
 * or >= nq) runs in one pass without the array, whatever its size.
 * Calls on one GPU share the array: calls that overlap in time on one GPU
 * (unordered streams) race and give undefined results; calls ordered on one
 * stream are safe.  The array's contents after a call are unspecified.
 */
qsa_status qsa_select_phase_noalloc(const float *q32, uint16_t *q16, int64_t q_tok_stride,
                                    const uint16_t *kblk, int64_t kblk_head_stride,
                                    int32_t *ids, int64_t ld_ids, float *vals,
                                    int32_t G, int32_t nq, int32_t H, int32_t D,
                                    int64_t n_kv, int32_t bs, int32_t k, int64_t q_chunk,
                                    uint32_t flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
