// qsa_noalloc.hip -- the select phase for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): qsa_select_phase_noalloc keeps the phase's score workspace in a
// file-scope device array instead of a caller buffer.
//
// The array is QSA_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held from the
// first call on that GPU until the process ends.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and passed to the phase's kernels like any workspace pointer; the array's
// name is never used as an address in host code.  Nothing in it has to start
// at zero: the scorer writes every score cell the selector reads.  With
// QSA_STREAM_SELECT, shapes the streaming scorer serves do not use it at all.
// Every call
// on a GPU uses the same array, so calls that overlap on one GPU (different
// streams, no ordering between them) race; calls on one stream do not.
#include "qsa.h"
#include "qsa_internal.h"

#include <mutex>

namespace {

constexpr int64_t kScratchBytes = QSA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte units");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The scratch array's address on the current device (looked up on the first
// call on that device), or null with *err set.
void *scratch_on_current_device(hipError_t *err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(g_once[dev], [dev] {
        void *p = nullptr;
        g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
    });
    *err = g_err[dev];
    return g_ptr[dev];
}

}  // namespace

extern "C" {

qsa_status qsa_select_phase_noalloc(const float *q32, uint16_t *q16, int64_t q_tok_stride,
                                    const uint16_t *kblk, int64_t kblk_head_stride,
                                    int32_t *ids, int64_t ld_ids, float *vals, int32_t G,
                                    int32_t nq, int32_t H, int32_t D, int64_t n_kv, int32_t bs,
                                    int32_t k, int64_t q_chunk, uint32_t flags, void *stream) {
    if (G < 0 || nq < 0 || n_kv < 0 || q_chunk < 0 ||
        (flags & ~(QSA_FORCE_TAIL | QSA_FUSED_SELECT | QSA_STREAM_SELECT)))
        return QSA_ERR_ARG;
    if (bs < 1) return QSA_ERR_UNSUPPORTED;
    // Rows of the workspace: nb scores rounded up to 32 floats, so that every
    // row starts on a 128-byte line.
    const int64_t nb = n_kv / bs + (n_kv % bs != 0);
    const int64_t ld_s = ((nb > 0 ? nb : 1) + 31) / 32 * 32;
    if (G == 0 || nq == 0) {
        // nothing to score or select; the phase itself checks the rest
        return qsa_select_phase(q32, q16, q_tok_stride, kblk, kblk_head_stride, nullptr, ld_s,
                                ids, ld_ids, vals, G, nq, H, D, n_kv, bs, k, 0, flags, stream);
    }
    // The streaming selection writes no score: where it serves the whole
    // shape in one pass (no q_chunk, or one of at least nq), the queries are
    // not chunked for the array (which is then only the phase's nominal
    // workspace, never written), whatever its size.
    if ((flags & QSA_STREAM_SELECT) && (q_chunk == 0 || q_chunk >= nq) && k > 0 && nb > 0) {
        const qsa::ScoreGeom geo{nullptr, q_tok_stride, kblk, kblk_head_stride, nullptr, ld_s,
                                 G, nq, H, D, n_kv / bs, 0.0f};
        if (qsa::stream_select_serves(geo, n_kv % bs != 0)) {
            hipError_t err = hipSuccess;
            void *ws = scratch_on_current_device(&err);
            if (!ws) return QSA_ERR_HIP;
            return qsa_select_phase(q32, q16, q_tok_stride, kblk, kblk_head_stride,
                                    static_cast<float *>(ws), ld_s, ids, ld_ids, vals, G, nq, H,
                                    D, n_kv, bs, k, 0, flags, stream);
        }
    }
    if (ld_s > kScratchBytes / 4 / G) return QSA_ERR_TOO_LARGE;   // not even one query fits
    const int64_t fit = kScratchBytes / (4 * G * ld_s);           // queries per pass
    int64_t qc = q_chunk > 0 ? q_chunk : fit;
    if (qc > nq) qc = nq;
    if (qc > fit) return QSA_ERR_TOO_LARGE;
    hipError_t err = hipSuccess;
    void *ws = scratch_on_current_device(&err);
    if (!ws) return QSA_ERR_HIP;
    return qsa_select_phase(q32, q16, q_tok_stride, kblk, kblk_head_stride,
                            static_cast<float *>(ws), ld_s, ids, ld_ids, vals, G, nq, H, D, n_kv,
                            bs, k, qc < nq ? qc : 0, flags, stream);
}

}  // extern "C"
