// qsa_api.hip -- the extern "C" boundary of libqsa.so (declared in qsa.h).
// Validates every argument before any HIP call, sizes the launches, and
// orchestrates the select phase on the caller's stream.  No allocation, no
// state, no synchronisation.  This file holds host code only: the launchers
// it calls live in the kernel files, so it also builds on its own, with
// host sanitizers, against stand-in launchers (the CPU test suite does).
#include "qsa.h"
#include "qsa_internal.h"

#include <string.h>

namespace qsa {

// Dispatch predicates (host only; declared in qsa_internal.h).
bool small_rows(const ScoreGeom &geo) {
    const int64_t wide_groups = (geo.nq + kGroupQueries - 1) / kGroupQueries;
    return static_cast<int64_t>(geo.G) * wide_groups < 256;
}

bool src32_ok(const float *q32, int64_t qts) {
    return reinterpret_cast<uintptr_t>(q32) % 16 == 0 && qts % 4 == 0;
}

// Workgroups per (KV head, query) row of the attention when a workspace is
// given: enough for one workgroup per CU over all rows, but no more than
// give each of a workgroup's 8 waves one 64-token chunk, and at most 64.
// Each split costs its own query staging, an 8-wave merge and a workspace
// round trip: at 256 rows of 64 chunks (8 heads, D = 128), two splits per row
// measured 95.5 us and four 111.9 us against 82.5 us for one.
int64_t attention_splits(int64_t rows, int32_t bs, int32_t k) {
    const int64_t chunks = static_cast<int64_t>(k) * ((static_cast<int64_t>(bs) + 63) / 64);
    int64_t sp = (256 + rows - 1) / rows;
    const int64_t by_chunks = (chunks + 7) / 8;
    if (sp > by_chunks) sp = by_chunks;
    if (sp > 64) sp = 64;
    return sp < 1 ? 1 : sp;
}

}  // namespace qsa

namespace {

using qsa::ScoreGeom;
using qsa::TopkGeom;

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
bool aligned4(const void *p) { return reinterpret_cast<uintptr_t>(p) % 4 == 0; }

// a*b + c without signed overflow; false when it would overflow int64.
bool mad_ok(int64_t a, int64_t b, int64_t c, int64_t *out) {
    int64_t m;
    if (__builtin_mul_overflow(a, b, &m)) return false;
    if (__builtin_add_overflow(m, c, out)) return false;
    return true;
}

struct ScoreCheck {
    int64_t nb = 0, nf = 0;
};

// Validation shared by qsa_block_scores and qsa_select_phase.
qsa_status check_scores_args(const void *q16, int64_t qts, const uint16_t *kblk, int64_t khs,
                             const float *scores, int64_t ld_s, int32_t G, int32_t nq, int32_t H,
                             int32_t D, int64_t n_kv, int32_t bs, ScoreCheck *out) {
    if (G < 0 || nq < 0 || n_kv < 0 || ld_s < 0 || qts < 0 || khs < 0) return QSA_ERR_ARG;
    if (bs < 1) return QSA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return QSA_ERR_UNSUPPORTED;
    if (H < 1 || H > 16) return QSA_ERR_UNSUPPORTED;
    const int64_t nb = n_kv / bs + (n_kv % bs != 0);
    out->nb = nb;
    out->nf = n_kv / bs;
    if (G == 0 || nq == 0 || nb == 0) return QSA_OK;   // nothing to read or write
    if (nb > 0x7fffffffLL) return QSA_ERR_UNSUPPORTED;
    if (!q16 || !kblk || !scores) return QSA_ERR_ARG;
    const int64_t row = static_cast<int64_t>(G) * H * D;
    if (qts < row) return QSA_ERR_ARG;
    int64_t tmp;
    if (!mad_ok(nb, D, 0, &tmp) || khs < tmp) return QSA_ERR_ARG;
    if (ld_s < nb) return QSA_ERR_ARG;
    // extents of every buffer must be addressable
    if (!mad_ok(static_cast<int64_t>(nq) - 1, qts, row, &tmp)) return QSA_ERR_ARG;
    if (!mad_ok(static_cast<int64_t>(G) - 1, khs, nb * D, &tmp)) return QSA_ERR_ARG;
    if (!mad_ok(static_cast<int64_t>(G) * nq - 1, ld_s, nb, &tmp)) return QSA_ERR_ARG;
    if (!aligned16(q16) || qts % 8 != 0) return QSA_ERR_UNSUPPORTED;
    if (!aligned16(kblk) || khs % 8 != 0) return QSA_ERR_UNSUPPORTED;
    if (!aligned4(scores)) return QSA_ERR_UNSUPPORTED;
    if (G > 65535) return QSA_ERR_UNSUPPORTED;
    return QSA_OK;
}

qsa_status check_topk_args(const float *scores, int64_t ld_s, int64_t rows, int32_t nb, int32_t k,
                           const int32_t *ids, int64_t ld_ids, const float *vals) {
    if (rows < 0 || nb < 0 || k < 0 || ld_s < 0 || ld_ids < 0) return QSA_ERR_ARG;
    if (k > QSA_MAX_K) return QSA_ERR_UNSUPPORTED;
    if (rows == 0 || k == 0) return QSA_OK;
    if (!ids || (nb > 0 && !scores)) return QSA_ERR_ARG;
    if (ld_ids < k) return QSA_ERR_ARG;
    if (nb > 0 && ld_s < nb) return QSA_ERR_ARG;
    int64_t tmp;
    if (!mad_ok(rows - 1, ld_ids, k, &tmp)) return QSA_ERR_ARG;
    if (nb > 0 && !mad_ok(rows - 1, ld_s, nb, &tmp)) return QSA_ERR_ARG;
    if (!aligned4(ids) || (vals && !aligned4(vals)) || (scores && !aligned4(scores)))
        return QSA_ERR_UNSUPPORTED;
    return QSA_OK;
}

qsa_status hip_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_ERR_HIP; }

// What the tail scorers add to the partial block's head sum.
float tail_addend(uint32_t flags) { return (flags & QSA_FORCE_TAIL) ? 1e9f : 0.0f; }

// Scores of every block (full blocks and the tail).  With q32 the queries
// are read as fp32 and converted on load (src32_ok holds), their fp16 bits
// written to q16w when it is set; with no full block the small scorer then
// scores the tail whatever the number of rows, since the standalone tail
// kernel reads fp16 queries only.
hipError_t run_scores(const ScoreGeom &geo, const ScoreCheck &c, hipStream_t s,
                      const float *q32 = nullptr, uint16_t *q16w = nullptr,
                      const qsa::FusedSelect *fs = nullptr, bool *selected = nullptr) {
    const bool tail = c.nb > c.nf;
    if (selected) *selected = false;
    if (c.nf > 0 && qsa::decode_rows(geo)) return qsa::launch_score_decode(geo, tail, s, q32, q16w);
    if (c.nf > 0) return qsa::launch_score_full(geo, tail, s, q32, q16w, fs, selected);
    if (!tail) return hipSuccess;
    if (q32 || qsa::small_rows(geo)) return qsa::launch_score_small(geo, true, s, q32, q16w);
    return qsa::launch_tail(geo, c.nf, s);
}

}  // namespace

extern "C" {

int qsa_abi_version(void) { return QSA_ABI_VERSION; }

const char *qsa_status_string(qsa_status s) {
    // A C caller may pass any int: read the bits rather than the enum value,
    // which C++ only defines for the enumerators' range.
    int v;
    memcpy(&v, &s, sizeof v);
    switch (v) {
        case QSA_OK: return "ok";
        case QSA_ERR_ARG: return "invalid argument (null pointer, negative size, stride or leading dimension too small)";
        case QSA_ERR_UNSUPPORTED: return "unsupported geometry (D not in {64,128}, H not in [1,16], k > 64, block size < 1, or misaligned pointer/stride)";
        case QSA_ERR_HIP: return "HIP runtime error at launch";
        case QSA_ERR_TOO_LARGE: return "the work does not fit the fixed scratch array of the no-allocation entry point (QSA_NOALLOC_SCRATCH_BYTES): pass a smaller q_chunk or use qsa_select_phase with a workspace";
    }
    return "unknown status";
}

qsa_status qsa_convert_f32_f16(const float *src, uint16_t *dst, int64_t n, void *stream) {
    if (n < 0) return QSA_ERR_ARG;
    if (n == 0) return QSA_OK;
    if (!src || !dst) return QSA_ERR_ARG;
    if (!aligned4(src) || reinterpret_cast<uintptr_t>(dst) % 2 != 0) return QSA_ERR_UNSUPPORTED;
    return hip_status(qsa::launch_convert(src, dst, n, static_cast<hipStream_t>(stream)));
}

qsa_status qsa_block_scores(const uint16_t *q16, int64_t q_tok_stride, const uint16_t *kblk,
                            int64_t kblk_head_stride, float *scores, int64_t ld_s, int32_t G,
                            int32_t nq, int32_t H, int32_t D, int64_t n_kv, int32_t bs,
                            uint32_t flags, void *stream) {
    if (flags & ~QSA_FORCE_TAIL) return QSA_ERR_ARG;
    ScoreCheck c;
    qsa_status st = check_scores_args(q16, q_tok_stride, kblk, kblk_head_stride, scores, ld_s, G,
                                      nq, H, D, n_kv, bs, &c);
    if (st != QSA_OK || G == 0 || nq == 0 || c.nb == 0) return st;
    ScoreGeom geo{q16, q_tok_stride, kblk, kblk_head_stride, scores, ld_s, G, nq, H, D, c.nf,
                  tail_addend(flags)};
    return hip_status(run_scores(geo, c, static_cast<hipStream_t>(stream)));
}

qsa_status qsa_select_topk(const float *scores, int64_t ld_s, int64_t rows, int32_t nb, int32_t k,
                           int32_t *ids, int64_t ld_ids, float *vals, void *stream) {
    qsa_status st = check_topk_args(scores, ld_s, rows, nb, k, ids, ld_ids, vals);
    if (st != QSA_OK || rows == 0 || k == 0) return st;
    TopkGeom geo{scores, ld_s, ids, ld_ids, vals, 1, rows, rows, rows, 0, nb, k};
    return hip_status(qsa::launch_topk(geo, static_cast<hipStream_t>(stream)));
}

qsa_status qsa_block_keys(const uint16_t *k_tok, int64_t tok_stride, uint16_t *kblk,
                          int64_t kblk_head_stride, int32_t G, int32_t D, int64_t n_kv,
                          int32_t bs, void *stream) {
    if (G < 0 || n_kv < 0 || tok_stride < 0 || kblk_head_stride < 0) return QSA_ERR_ARG;
    if (bs < 1 || bs > QSA_BLOCK_KEYS_MAX_BS) return QSA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return QSA_ERR_UNSUPPORTED;
    if (G == 0 || n_kv == 0) return QSA_OK;
    if (!k_tok || !kblk) return QSA_ERR_ARG;
    const int64_t nb = n_kv / bs + (n_kv % bs != 0);
    int64_t tmp;
    if (tok_stride < static_cast<int64_t>(G) * D) return QSA_ERR_ARG;
    if (!mad_ok(nb, D, 0, &tmp) || kblk_head_stride < tmp) return QSA_ERR_ARG;
    if (!mad_ok(n_kv - 1, tok_stride, static_cast<int64_t>(G) * D, &tmp)) return QSA_ERR_ARG;
    if (!mad_ok(static_cast<int64_t>(G) - 1, kblk_head_stride, nb * D, &tmp)) return QSA_ERR_ARG;
    if (!aligned16(k_tok) || tok_stride % 8 != 0) return QSA_ERR_UNSUPPORTED;
    if (!aligned16(kblk) || kblk_head_stride % 8 != 0) return QSA_ERR_UNSUPPORTED;
    return hip_status(qsa::launch_block_keys(k_tok, tok_stride, kblk, kblk_head_stride, G, D, n_kv,
                                             bs, static_cast<hipStream_t>(stream)));
}

int64_t qsa_sparse_attention_ws_floats(int32_t G, int32_t nq, int32_t H, int32_t D, int32_t bs,
                                       int32_t k) {
    if (G <= 0 || nq <= 0 || H < 1 || H > 16 || (D != 64 && D != 128) || bs < 1 || k < 1 ||
        k > QSA_MAX_K)
        return 0;
    const int64_t rows = static_cast<int64_t>(G) * nq;
    const int64_t sp = qsa::attention_splits(rows, bs, k);
    return sp > 1 ? sp * rows * H * (2 + D) : 0;
}

qsa_status qsa_sparse_attention(const uint16_t *q16, int64_t q_tok_stride, const uint16_t *k_tok,
                                const uint16_t *v_tok, int64_t kv_tok_stride, const int32_t *ids,
                                int64_t ld_ids, float *out, int64_t out_tok_stride, int32_t G,
                                int32_t nq, int32_t H, int32_t D, int64_t n_kv, int32_t bs,
                                int32_t k, float *ws, int64_t ws_floats, void *stream) {
    if (G < 0 || nq < 0 || n_kv < 0 || k < 0 || q_tok_stride < 0 || kv_tok_stride < 0 ||
        ld_ids < 0 || out_tok_stride < 0 || ws_floats < 0)
        return QSA_ERR_ARG;
    if (bs < 1) return QSA_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return QSA_ERR_UNSUPPORTED;
    if (H < 1 || H > 16) return QSA_ERR_UNSUPPORTED;
    if (k > QSA_MAX_K) return QSA_ERR_UNSUPPORTED;
    if (G == 0 || nq == 0) return QSA_OK;
    if (!q16 || !out || (k > 0 && !ids)) return QSA_ERR_ARG;
    if (n_kv > 0 && (!k_tok || !v_tok)) return QSA_ERR_ARG;
    const int64_t row = static_cast<int64_t>(G) * H * D;
    if (q_tok_stride < row || out_tok_stride < row) return QSA_ERR_ARG;
    if (ld_ids < k) return QSA_ERR_ARG;
    int64_t tmp;
    if (!mad_ok(static_cast<int64_t>(nq) - 1, q_tok_stride, row, &tmp)) return QSA_ERR_ARG;
    if (!mad_ok(static_cast<int64_t>(nq) - 1, out_tok_stride, row, &tmp)) return QSA_ERR_ARG;
    if (!mad_ok(static_cast<int64_t>(G) * nq - 1, ld_ids, k, &tmp)) return QSA_ERR_ARG;
    if (n_kv > 0) {
        if (kv_tok_stride < static_cast<int64_t>(G) * D) return QSA_ERR_ARG;
        if (!mad_ok(n_kv - 1, kv_tok_stride, static_cast<int64_t>(G) * D, &tmp)) return QSA_ERR_ARG;
        if (!aligned16(k_tok) || !aligned16(v_tok) || kv_tok_stride % 8 != 0)
            return QSA_ERR_UNSUPPORTED;
        // a chunk's 64 value rows are addressed with 32-bit byte offsets
        if (kv_tok_stride > QSA_ATTENTION_MAX_KV_STRIDE) return QSA_ERR_UNSUPPORTED;
    }
    if (reinterpret_cast<uintptr_t>(q16) % 2 != 0 || !aligned4(out) || (ids && !aligned4(ids)) ||
        (ws && !aligned4(ws)))
        return QSA_ERR_UNSUPPORTED;
    return hip_status(qsa::launch_attention(q16, q_tok_stride, k_tok, v_tok, kv_tok_stride, ids,
                                            ld_ids, out, out_tok_stride, G, nq, H, D, n_kv, bs, k,
                                            ws, ws ? ws_floats : 0,
                                            static_cast<hipStream_t>(stream)));
}

qsa_status qsa_select_phase(const float *q32, uint16_t *q16, int64_t q_tok_stride,
                            const uint16_t *kblk, int64_t kblk_head_stride, float *scores_ws,
                            int64_t ld_s, int32_t *ids, int64_t ld_ids, float *vals, int32_t G,
                            int32_t nq, int32_t H, int32_t D, int64_t n_kv, int32_t bs, int32_t k,
                            int64_t q_chunk, uint32_t flags, void *stream) {
    if (q_chunk < 0 || (flags & ~(QSA_FORCE_TAIL | QSA_FUSED_SELECT | QSA_STREAM_SELECT)))
        return QSA_ERR_ARG;
    const int64_t qc = (q_chunk > 0 && q_chunk < nq) ? q_chunk : nq;
    ScoreCheck c;
    // scores are validated for the chunk-sized workspace; the query source
    // is the fp16 buffer when there is one, else the fp32 queries
    const void *qsrc = q16 ? static_cast<const void *>(q16) : static_cast<const void *>(q32);
    qsa_status st = check_scores_args(qsrc, q_tok_stride, kblk, kblk_head_stride, scores_ws, ld_s,
                                      G, static_cast<int32_t>(qc), H, D, n_kv, bs, &c);
    if (st != QSA_OK) return st;
    if (G == 0 || nq == 0) return QSA_OK;
    // the whole query tensor (not only one chunk of it) must be addressable
    int64_t qext = 0;
    if (!mad_ok(static_cast<int64_t>(nq) - 1, q_tok_stride, static_cast<int64_t>(G) * H * D,
                &qext))
        return QSA_ERR_ARG;
    const int64_t rows = static_cast<int64_t>(G) * nq;
    st = check_topk_args(scores_ws, ld_s, rows, static_cast<int32_t>(c.nb), k, ids, ld_ids, vals);
    if (st != QSA_OK) return st;
    if (q32) {
        if (!aligned4(q32) || reinterpret_cast<uintptr_t>(q16) % 2 != 0)
            return QSA_ERR_UNSUPPORTED;
        // without an fp16 buffer the scorers must read the fp32 rows directly
        if (!q16 && !qsa::src32_ok(q32, q_tok_stride)) return QSA_ERR_UNSUPPORTED;
    } else if (!q16) {
        return QSA_ERR_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);

    for (int64_t t0 = 0; t0 < nq; t0 += qc) {
        const int32_t n = static_cast<int32_t>((nq - t0 < qc) ? nq - t0 : qc);
        const int64_t qoff = t0 * q_tok_stride;
        uint16_t *q16c = q16 ? q16 + qoff : nullptr;   // may be null when nb == 0
        ScoreGeom geo{q16c, q_tok_stride, kblk, kblk_head_stride, scores_ws, ld_s, G, n, H, D,
                      c.nf, tail_addend(flags)};
        // With 16-byte aligned fp32 queries the scorer reads them itself,
        // converts them on load and writes this chunk's rows of the fp16
        // buffer (if any), so the conversion needs no launch of its own;
        // otherwise the conversion kernel writes exactly the chunk's token
        // rows (G*H*D elements each) first.
        const bool fused = q32 && c.nb > 0 && qsa::src32_ok(q32 + qoff, q_tok_stride);
        if (q32 && !fused && q16c) {
            hipError_t e = qsa::launch_convert_rows(q32 + qoff, q16c, n,
                                                    static_cast<int64_t>(G) * H * D, q_tok_stride, s);
            if (e != hipSuccess) return QSA_ERR_HIP;
        }
        // with QSA_STREAM_SELECT or QSA_FUSED_SELECT the shapes the
        // streaming or fused scorer serves are selected inside the scorer's
        // launch
        const qsa::FusedSelect fsel{ids, ld_ids, vals, k, nq, t0, (flags & QSA_STREAM_SELECT) != 0,
                                    (flags & QSA_FUSED_SELECT) != 0};
        const qsa::FusedSelect *fs =
            (flags & (QSA_FUSED_SELECT | QSA_STREAM_SELECT)) && k > 0 ? &fsel : nullptr;
        bool selected = false;
        if (c.nb > 0) {
            hipError_t e = fused ? run_scores(geo, c, s, q32 + qoff, q16c, fs, &selected)
                                 : run_scores(geo, c, s, nullptr, nullptr, fs, &selected);
            if (e != hipSuccess) return QSA_ERR_HIP;
        }
        if (k > 0 && !selected) {
            // the scorer wrote this chunk's rows at g*n + t' (n = rows in the
            // chunk); in one pass over all rows that is the output's row
            // order too, and the selector sees one flat group of rows
            const int64_t rows = static_cast<int64_t>(G) * n;
            TopkGeom tg = n == nq
                ? TopkGeom{scores_ws, ld_s, ids, ld_ids, vals, 1, rows, rows, rows, 0,
                           static_cast<int32_t>(c.nb), k}
                : TopkGeom{scores_ws, ld_s, ids, ld_ids, vals, G, n, n, nq, t0,
                           static_cast<int32_t>(c.nb), k};
            hipError_t e = qsa::launch_topk(tg, s);
            if (e != hipSuccess) return QSA_ERR_HIP;
        }
    }
    return QSA_OK;
}

}  // extern "C"
