// Test driver: the host side of libqsa's C ABI (csrc/qsa_api.hip, compiled
// for the host with AddressSanitizer and UndefinedBehaviorSanitizer) linked
// against stand-in launchers that record what they were asked to launch.
// Built and run by the CPU test suite; exit status 0 means every check passed
// and no sanitizer fired.
//
// Checked: every refusal returns its documented status and launches nothing
// (the pages require the host entry to refuse unsupported geometry:
// Strata pull request #228, part 1, the "opt-in, with an honest fallback"
// paragraph), empty calls are OK without a launch, and valid calls reach the
// launchers with the sizes the header documents (the query-chunk loop of the
// phase, the fused conversion, the flat or grouped selector rows).  No device
// memory is touched: the pointers are fake, aligned addresses.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "qsa.h"
#include "qsa_internal.h"

namespace {

struct Launch {
    char kind;   // 'f' full scorer, 's' small scorer, 'd' decode scorer, 't' tail, 'k' top-k,
                 // 'c' convert, 'r' rows, 'b' block keys, 'a' attention, 'F' fused selection
    int64_t a, b, c;
};
std::vector<Launch> g_launches;

}  // namespace

namespace qsa {
hipError_t launch_score_full(const ScoreGeom &g, bool tail, hipStream_t, const float *q32,
                             uint16_t *, const FusedSelect *fs, bool *selected) {
    // the real launcher hands few rows to the small scorer: bit 4 records it
    g_launches.push_back({'f', g.nq, g.nf, (tail ? 1 : 0) + (q32 ? 2 : 0) + (small_rows(g) ? 4 : 0) +
                                              (g.tail_add == 1e9f ? 8 : 0)});
    // a fused selection request: 'F' records where the ids go; this stand-in
    // takes it for 4096 or more query rows per pass (the real launcher
    // decides by shape)
    if (selected) *selected = false;
    if (fs) {
        g_launches.push_back({'F', fs->dst_group_rows, fs->dst_row0,
                              fs->k | (fs->stream ? 0x100 : 0) | (fs->fused ? 0x200 : 0)});
        if (selected) *selected = g.nq >= 4096;
    }
    return hipSuccess;
}
bool decode_rows(const ScoreGeom &g) {   // the rule of qsa_decode.hip
    const int np = (g.H + 1) / 2;
    const int pairs = np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : 8;
    return g.nq > 0 && g.nq <= 16 / pairs && g.nf > 0;
}
hipError_t launch_score_decode(const ScoreGeom &g, bool tail, hipStream_t, const float *q32,
                               uint16_t *) {
    g_launches.push_back({'d', g.nq, g.nf, (tail ? 1 : 0) + (q32 ? 2 : 0) + (g.tail_add == 1e9f ? 8 : 0)});
    return hipSuccess;
}
hipError_t launch_score_small(const ScoreGeom &g, bool tail, hipStream_t, const float *q32,
                              uint16_t *) {
    g_launches.push_back({'s', g.nq, g.nf, (tail ? 1 : 0) + (q32 ? 2 : 0) + (g.tail_add == 1e9f ? 8 : 0)});
    return hipSuccess;
}
hipError_t launch_tail(const ScoreGeom &g, int64_t b, hipStream_t) {
    g_launches.push_back({'t', g.nq, b, g.tail_add == 1e9f ? 8 : 0});
    return hipSuccess;
}
hipError_t launch_topk(const TopkGeom &g, hipStream_t) {
    g_launches.push_back({'k', g.n_groups * g.rows_per_group, g.dst_row0, g.nb});
    return hipSuccess;
}
hipError_t launch_convert(const float *, uint16_t *, int64_t n, hipStream_t) {
    g_launches.push_back({'c', n, 0, 0});
    return hipSuccess;
}
hipError_t launch_block_keys(const uint16_t *, int64_t, uint16_t *, int64_t, int32_t G, int32_t D,
                             int64_t n_kv, int32_t bs, hipStream_t) {
    g_launches.push_back({'b', G * 1000 + D, n_kv, bs});
    return hipSuccess;
}
hipError_t launch_attention(const uint16_t *, int64_t, const uint16_t *, const uint16_t *, int64_t,
                            const int32_t *, int64_t, float *, int64_t, int32_t G, int32_t nq,
                            int32_t H, int32_t D, int64_t n_kv, int32_t bs, int32_t k, float *,
                            int64_t, hipStream_t) {
    g_launches.push_back({'a', static_cast<int64_t>(G) * nq, n_kv, H * 1000 + D + k * 100000 + bs * 0});
    return hipSuccess;
}
hipError_t launch_convert_rows(const float *, uint16_t *, int64_t rows, int64_t row_len,
                               int64_t, hipStream_t) {
    g_launches.push_back({'r', rows, row_len, 0});
    return hipSuccess;
}
}  // namespace qsa

static int failures = 0;
#define CHECK(c, ...)                                                \
    do {                                                             \
        if (!(c)) {                                                  \
            fprintf(stderr, "FAIL line %d: ", __LINE__);             \
            fprintf(stderr, __VA_ARGS__);                            \
            fprintf(stderr, "\n");                                   \
            ++failures;                                              \
        }                                                            \
    } while (0)

static uint16_t *const H16 = reinterpret_cast<uint16_t *>(uintptr_t(0x10000));
static float *const F32 = reinterpret_cast<float *>(uintptr_t(0x20000));
static int32_t *const I32 = reinterpret_cast<int32_t *>(uintptr_t(0x30000));

struct SArgs {
    const uint16_t *q16 = H16;
    int64_t qts = 8 * 128;
    const uint16_t *kblk = H16;
    int64_t khs = 64 * 128;
    float *scores = F32;
    int64_t ld_s = 64;
    int32_t G = 1, nq = 256, H = 8, D = 128;
    int64_t n_kv = 4096;
    int32_t bs = 64;
    uint32_t flags = 0;
    qsa_status call() const {
        return qsa_block_scores(q16, qts, kblk, khs, scores, ld_s, G, nq, H, D, n_kv, bs, flags,
                                nullptr);
    }
};

struct PArgs {
    const float *q32 = F32;
    uint16_t *q16 = H16;
    int64_t qts = 8 * 128;
    const uint16_t *kblk = H16;
    int64_t khs = 64 * 128;
    float *ws = F32;
    int64_t ld_s = 64;
    int32_t *ids = I32;
    int64_t ld_ids = 16;
    float *vals = nullptr;
    int32_t G = 1, nq = 256, H = 8, D = 128;
    int64_t n_kv = 4096;
    int32_t bs = 64, k = 16;
    int64_t q_chunk = 0;
    uint32_t flags = 0;
    qsa_status call() const {
        return qsa_select_phase(q32, q16, qts, kblk, khs, ws, ld_s, ids, ld_ids, vals, G, nq, H, D,
                                n_kv, bs, k, q_chunk, flags, nullptr);
    }
};

template <class F>
static void expect(const char *name, qsa_status want, F call, size_t launches) {
    g_launches.clear();
    const qsa_status got = call();
    CHECK(got == want, "%s: status %d, expected %d", name, int(got), int(want));
    CHECK(g_launches.size() == launches, "%s: %zu launches, expected %zu", name,
          g_launches.size(), launches);
}

int main() {
    // ---- qsa_block_scores ------------------------------------------------
    {
        SArgs a;
        expect("scores ok", QSA_OK, [&] { return a.call(); }, 1);
        CHECK(g_launches.size() == 1 && g_launches[0].kind == 'f' && g_launches[0].b == 64 &&
                  (g_launches[0].c & 4) && !(g_launches[0].c & 1),
              "256 queries of one KV head: the small scorer over 64 full blocks, no tail");
        SArgs w;
        w.G = 4;
        w.nq = 16384;
        w.n_kv = 131077;
        w.khs = 2049 * 128;
        w.ld_s = 2080;
        w.qts = 4 * 8 * 128;
        expect("prefill scores", QSA_OK, [&] { return w.call(); }, 1);
        CHECK(g_launches[0].kind == 'f' && g_launches[0].b == 2048 && g_launches[0].c == 1,
              "the prefill chunk takes the wide scorer with the tail");
        SArgs t = a;
        t.n_kv = 40;
        t.G = 4;
        t.nq = 16384;
        t.qts = 4 * 8 * 128;
        t.ld_s = 1;
        SArgs d = a;   // a decode step: one query of each of 8 KV heads, 2048 blocks + a tail
        d.G = 8;
        d.nq = 1;
        d.qts = 8 * 8 * 128;
        d.n_kv = 131109;
        d.khs = 2049 * 128;
        d.ld_s = 2049;
        d.flags = QSA_FORCE_TAIL;
        expect("decode scores", QSA_OK, [&] { return d.call(); }, 1);
        CHECK(g_launches[0].kind == 'd' && g_launches[0].b == 2048 && g_launches[0].c == (1 | 8),
              "a decode step takes the decode scorer, tail and forced rule included");
        d.nq = 5;   // past one row block of 4 queries at H = 8
        expect("five queries per KV head", QSA_OK, [&] { return d.call(); }, 1);
        CHECK(g_launches[0].kind == 'f' && (g_launches[0].c & 4), "five queries take the small scorer");
        expect("tail only, many rows", QSA_OK, [&] { return t.call(); }, 1);
        CHECK(g_launches[0].kind == 't' && g_launches[0].b == 0 && g_launches[0].c == 0,
              "standalone tail of block 0, nothing added");
        t.flags = QSA_FORCE_TAIL;
        expect("tail only, forced", QSA_OK, [&] { return t.call(); }, 1);
        CHECK(g_launches[0].kind == 't' && g_launches[0].c == 8, "the tail kernel adds 1e9");
        w.flags = QSA_FORCE_TAIL;
        expect("prefill scores, forced tail", QSA_OK, [&] { return w.call(); }, 1);
        CHECK(g_launches[0].kind == 'f' && g_launches[0].c == (1 | 8),
              "the wide scorer's tail adds 1e9");
    }
    struct SCase {
        const char *name;
        void (*set)(SArgs &);
        qsa_status want;
    };
    const SCase scases[] = {
        {"D=96", [](SArgs &a) { a.D = 96; }, QSA_ERR_UNSUPPORTED},
        {"flags=2", [](SArgs &a) { a.flags = 2; }, QSA_ERR_ARG},
        {"flags=~0", [](SArgs &a) { a.flags = ~0u; }, QSA_ERR_ARG},
        {"H=0", [](SArgs &a) { a.H = 0; }, QSA_ERR_UNSUPPORTED},
        {"H=17", [](SArgs &a) { a.H = 17; }, QSA_ERR_UNSUPPORTED},
        {"bs=0", [](SArgs &a) { a.bs = 0; }, QSA_ERR_UNSUPPORTED},
        {"n_kv<0", [](SArgs &a) { a.n_kv = -1; }, QSA_ERR_ARG},
        {"G<0", [](SArgs &a) { a.G = -1; }, QSA_ERR_ARG},
        {"nq<0", [](SArgs &a) { a.nq = -5; }, QSA_ERR_ARG},
        {"q16 null", [](SArgs &a) { a.q16 = nullptr; }, QSA_ERR_ARG},
        {"kblk null", [](SArgs &a) { a.kblk = nullptr; }, QSA_ERR_ARG},
        {"scores null", [](SArgs &a) { a.scores = nullptr; }, QSA_ERR_ARG},
        {"ld_s<nb", [](SArgs &a) { a.ld_s = 63; }, QSA_ERR_ARG},
        {"qts small", [](SArgs &a) { a.qts = 8 * 128 - 8; }, QSA_ERR_ARG},
        {"khs small", [](SArgs &a) { a.khs = 63 * 128; }, QSA_ERR_ARG},
        {"q16 misaligned", [](SArgs &a) { a.q16 = H16 + 1; }, QSA_ERR_UNSUPPORTED},
        {"qts misaligned", [](SArgs &a) { a.qts = 8 * 128 + 4; }, QSA_ERR_UNSUPPORTED},
        {"kblk misaligned", [](SArgs &a) { a.kblk = H16 + 4; }, QSA_ERR_UNSUPPORTED},
        {"scores extent overflow", [](SArgs &a) { a.ld_s = int64_t(1) << 62; a.nq = 8; },
         QSA_ERR_ARG},
        {"query extent overflow", [](SArgs &a) { a.qts = int64_t(1) << 60; }, QSA_ERR_ARG},
        {"G too large", [](SArgs &a) { a.G = 70000; a.khs = 64 * 128; a.qts = int64_t(70000) * 1024; },
         QSA_ERR_UNSUPPORTED},
    };
    for (const SCase &c : scases) {
        SArgs a;
        c.set(a);
        expect(c.name, c.want, [&] { return a.call(); }, 0);
    }
    {
        SArgs a;
        a.n_kv = 0;
        a.q16 = nullptr;
        a.kblk = nullptr;
        a.scores = nullptr;
        expect("n_kv=0, no pointers", QSA_OK, [&] { return a.call(); }, 0);
        SArgs b;
        b.nq = 0;
        expect("nq=0", QSA_OK, [&] { return b.call(); }, 0);
    }

    // ---- qsa_select_topk ---------------------------------------------------
    expect("topk ok", QSA_OK,
           [] { return qsa_select_topk(F32, 2048, 256, 2048, 64, I32, 64, F32, nullptr); }, 1);
    expect("topk k>64", QSA_ERR_UNSUPPORTED,
           [] { return qsa_select_topk(F32, 2048, 256, 2048, 65, I32, 65, nullptr, nullptr); }, 0);
    expect("topk k<0", QSA_ERR_ARG,
           [] { return qsa_select_topk(F32, 2048, 256, 2048, -1, I32, 64, nullptr, nullptr); }, 0);
    expect("topk ids null", QSA_ERR_ARG,
           [] { return qsa_select_topk(F32, 2048, 256, 2048, 64, nullptr, 64, nullptr, nullptr); }, 0);
    expect("topk ld_ids<k", QSA_ERR_ARG,
           [] { return qsa_select_topk(F32, 2048, 256, 2048, 64, I32, 63, nullptr, nullptr); }, 0);
    expect("topk ld_s<nb", QSA_ERR_ARG,
           [] { return qsa_select_topk(F32, 2047, 256, 2048, 64, I32, 64, nullptr, nullptr); }, 0);
    expect("topk vals misaligned", QSA_ERR_UNSUPPORTED, [] {
        return qsa_select_topk(F32, 2048, 256, 2048, 64, I32, 64,
                               reinterpret_cast<float *>(uintptr_t(0x20001)), nullptr);
    }, 0);
    expect("topk rows overflow", QSA_ERR_ARG, [] {
        return qsa_select_topk(F32, int64_t(1) << 62, 16, 2048, 64, I32, 64, nullptr, nullptr);
    }, 0);
    expect("topk k=0", QSA_OK,
           [] { return qsa_select_topk(F32, 2048, 256, 2048, 0, nullptr, 0, nullptr, nullptr); }, 0);
    expect("topk nb=0 pads", QSA_OK,
           [] { return qsa_select_topk(nullptr, 0, 256, 0, 8, I32, 8, nullptr, nullptr); }, 1);

    // ---- qsa_block_keys -----------------------------------------------------
    expect("keys ok", QSA_OK,
           [] { return qsa_block_keys(H16, 4 * 128, H16, 2049 * 128, 4, 128, 131077, 64, nullptr); }, 1);
    CHECK(g_launches[0].kind == 'b' && g_launches[0].a == 4128 && g_launches[0].b == 131077,
          "block keys of 4 KV heads, D = 128");
    expect("keys bs>8192", QSA_ERR_UNSUPPORTED,
           [] { return qsa_block_keys(H16, 512, H16, 128, 4, 128, 8193, 8193, nullptr); }, 0);
    expect("keys D=32", QSA_ERR_UNSUPPORTED,
           [] { return qsa_block_keys(H16, 512, H16, 2049 * 32, 4, 32, 131077, 64, nullptr); }, 0);
    expect("keys khs small", QSA_ERR_ARG,
           [] { return qsa_block_keys(H16, 512, H16, 2048 * 128, 4, 128, 131077, 64, nullptr); }, 0);
    expect("keys misaligned", QSA_ERR_UNSUPPORTED,
           [] { return qsa_block_keys(H16 + 1, 512, H16, 2049 * 128, 4, 128, 131077, 64, nullptr); }, 0);
    expect("keys empty", QSA_OK,
           [] { return qsa_block_keys(nullptr, 512, nullptr, 0, 4, 128, 0, 64, nullptr); }, 0);

    // ---- qsa_sparse_attention -----------------------------------------------
    expect("attention ok", QSA_OK, [] {
        return qsa_sparse_attention(H16, 1024, H16, H16, 128, I32, 64, F32, 1024, 1, 256, 8, 128,
                                    131072, 64, 64, nullptr, 0, nullptr);
    }, 1);
    CHECK(g_launches[0].kind == 'a' && g_launches[0].a == 256 && g_launches[0].b == 131072,
          "attention over 256 rows");
    expect("attention n_kv=0 still writes zeros", QSA_OK, [] {
        return qsa_sparse_attention(H16, 1024, nullptr, nullptr, 0, I32, 64, F32, 1024, 1, 256, 8,
                                    128, 0, 64, 64, nullptr, 0, nullptr);
    }, 1);
    expect("attention H=17", QSA_ERR_UNSUPPORTED, [] {
        return qsa_sparse_attention(H16, 17 * 128, H16, H16, 128, I32, 64, F32, 17 * 128, 1, 256,
                                    17, 128, 131072, 64, 64, nullptr, 0, nullptr);
    }, 0);
    expect("attention kv misaligned", QSA_ERR_UNSUPPORTED, [] {
        return qsa_sparse_attention(H16, 1024, H16 + 4, H16, 128, I32, 64, F32, 1024, 1, 256, 8,
                                    128, 131072, 64, 64, nullptr, 0, nullptr);
    }, 0);
    expect("attention nq=0", QSA_OK, [] {
        return qsa_sparse_attention(nullptr, 0, nullptr, nullptr, 0, nullptr, 0, nullptr, 0, 1, 0,
                                    8, 128, 0, 64, 64, nullptr, 0, nullptr);
    }, 0);

    // ---- qsa_convert_f32_f16 -----------------------------------------------
    expect("convert ok", QSA_OK, [] { return qsa_convert_f32_f16(F32, H16, 1000, nullptr); }, 1);
    expect("convert n<0", QSA_ERR_ARG, [] { return qsa_convert_f32_f16(F32, H16, -1, nullptr); }, 0);
    expect("convert null", QSA_ERR_ARG, [] { return qsa_convert_f32_f16(nullptr, H16, 8, nullptr); }, 0);
    expect("convert misaligned", QSA_ERR_UNSUPPORTED, [] {
        return qsa_convert_f32_f16(reinterpret_cast<float *>(uintptr_t(0x20002)), H16, 8, nullptr);
    }, 0);
    expect("convert n=0", QSA_OK, [] { return qsa_convert_f32_f16(nullptr, nullptr, 0, nullptr); }, 0);

    // ---- qsa_select_phase ----------------------------------------------------
    {
        PArgs a;
        a.q16 = nullptr;   // 16-byte aligned fp32 rows: converted by the scorer on load
        expect("phase fused", QSA_OK, [&] { return a.call(); }, 2);
        CHECK(g_launches[0].kind == 'f' && (g_launches[0].c & 2) && g_launches[1].kind == 'k' &&
                  g_launches[1].a == 256 && !(g_launches[0].c & 8),
              "fused phase: scorer with fp32 queries, then one flat selector launch");
        a.flags = QSA_FORCE_TAIL;
        a.n_kv = 4096 + 7;   // 64 full blocks and a 7-token tail
        a.khs = 65 * 128;
        a.ld_s = 65;
        expect("phase forced tail", QSA_OK, [&] { return a.call(); }, 2);
        CHECK(g_launches[0].kind == 'f' && (g_launches[0].c & 1) && (g_launches[0].c & 8),
              "forced tail: the phase's scorer adds 1e9 to the partial block");
        a.flags = QSA_FUSED_SELECT;
        expect("phase fused select, not taken", QSA_OK, [&] { return a.call(); }, 3);
        CHECK(g_launches[1].kind == 'F' && g_launches[1].a == 256 && g_launches[1].b == 0 &&
                  g_launches[1].c == (16 | 0x200) && g_launches[2].kind == 'k',
              "a fused request the scorer declines is followed by the selector launch");
        a.flags = QSA_STREAM_SELECT;
        expect("phase stream select, not taken", QSA_OK, [&] { return a.call(); }, 3);
        CHECK(g_launches[1].kind == 'F' && g_launches[1].c == (16 | 0x100) &&
                  g_launches[2].kind == 'k',
              "a streaming request the scorer declines is followed by the selector launch");
        a.flags = QSA_STREAM_SELECT | QSA_FUSED_SELECT | QSA_FORCE_TAIL;
        expect("phase all flags", QSA_OK, [&] { return a.call(); }, 3);
        CHECK(g_launches[0].kind == 'f' && (g_launches[0].c & 8) && g_launches[1].kind == 'F' &&
                  g_launches[1].c == (16 | 0x300),
              "every flag reaches the scorer");
        PArgs f;
        f.q16 = nullptr;
        f.flags = QSA_FUSED_SELECT;
        f.G = 2;
        f.nq = 8192;
        f.qts = 2 * 8 * 128;
        f.q_chunk = 4096;
        expect("phase fused select, chunks", QSA_OK, [&] { return f.call(); }, 4);
        CHECK(g_launches[0].kind == 'f' && g_launches[1].kind == 'F' && g_launches[1].a == 8192 &&
                  g_launches[1].b == 0 && g_launches[2].kind == 'f' && g_launches[3].kind == 'F' &&
                  g_launches[3].b == 4096,
              "fused chunks: the ids of chunk j go to query rows 4096*j onwards, no selector launch");
        PArgs b;
        b.q32 = reinterpret_cast<float *>(uintptr_t(0x20004));   // 4-byte aligned only
        expect("phase separate conversion", QSA_OK, [&] { return b.call(); }, 3);
        CHECK(g_launches[0].kind == 'r' && g_launches[0].a == 256 && g_launches[0].b == 1024,
              "conversion of the 256 token rows of 1024 elements first");
        PArgs c;
        c.q16 = nullptr;
        c.G = 3;
        c.nq = 150;
        c.q_chunk = 64;
        c.qts = 3 * 8 * 128;
        c.ld_ids = 16;
        expect("phase chunks", QSA_OK, [&] { return c.call(); }, 6);
        const int64_t want_rows[3] = {64, 64, 22};
        for (int j = 0; j < 3; ++j) {
            CHECK(g_launches[2 * j].kind == 'f' && g_launches[2 * j].a == want_rows[j],
                  "chunk %d scores %lld queries", j, (long long)want_rows[j]);
            CHECK(g_launches[2 * j + 1].kind == 'k' && g_launches[2 * j + 1].a == 3 * want_rows[j] &&
                      g_launches[2 * j + 1].b == 64 * j,
                  "chunk %d selects its rows of every KV head into row %d onwards", j, 64 * j);
        }
        PArgs d;
        d.n_kv = 0;
        d.ld_s = 1;
        expect("phase n_kv=0", QSA_OK, [&] { return d.call(); }, 2);
        CHECK(g_launches[0].kind == 'r' && g_launches[1].kind == 'k' && g_launches[1].c == 0,
              "n_kv = 0: the kept fp16 copy is converted, the selector pads");
    }
    struct PCase {
        const char *name;
        void (*set)(PArgs &);
        qsa_status want;
    };
    const PCase pcases[] = {
        {"q_chunk<0", [](PArgs &a) { a.q_chunk = -1; }, QSA_ERR_ARG},
        {"flags=8", [](PArgs &a) { a.flags = 8; }, QSA_ERR_ARG},
        {"k>64", [](PArgs &a) { a.k = 65; a.ld_ids = 65; }, QSA_ERR_UNSUPPORTED},
        {"D=80", [](PArgs &a) { a.D = 80; }, QSA_ERR_UNSUPPORTED},
        {"ids null", [](PArgs &a) { a.ids = nullptr; }, QSA_ERR_ARG},
        {"no queries", [](PArgs &a) { a.q16 = nullptr; a.q32 = nullptr; }, QSA_ERR_ARG},
        {"ws null", [](PArgs &a) { a.ws = nullptr; }, QSA_ERR_ARG},
        {"ld_ids<k", [](PArgs &a) { a.ld_ids = 8; }, QSA_ERR_ARG},
        {"ld_s<nb", [](PArgs &a) { a.ld_s = 10; }, QSA_ERR_ARG},
        {"q32 misaligned", [](PArgs &a) { a.q32 = reinterpret_cast<float *>(uintptr_t(0x20002)); },
         QSA_ERR_UNSUPPORTED},
        {"H=20", [](PArgs &a) { a.H = 20; }, QSA_ERR_UNSUPPORTED},
        {"no fp16 buffer, rows 4-byte aligned",
         [](PArgs &a) { a.q16 = nullptr; a.q32 = reinterpret_cast<float *>(uintptr_t(0x20004)); },
         QSA_ERR_UNSUPPORTED},
        {"no fp16 buffer, odd stride", [](PArgs &a) { a.q16 = nullptr; a.qts = 8 * 128 + 2; },
         QSA_ERR_UNSUPPORTED},
        {"query extent overflow", [](PArgs &a) { a.qts = int64_t(1) << 56; }, QSA_ERR_ARG},
    };
    for (const PCase &c : pcases) {
        PArgs a;
        c.set(a);
        expect(c.name, c.want, [&] { return a.call(); }, 0);
    }
    {
        PArgs a;
        a.nq = 0;
        expect("phase nq=0", QSA_OK, [&] { return a.call(); }, 0);
        PArgs b;
        b.G = 0;
        expect("phase G=0", QSA_OK, [&] { return b.call(); }, 0);
    }
    for (int s = 0; s <= 3; ++s) CHECK(qsa_status_string(static_cast<qsa_status>(s)) != nullptr, "status string");
    // (a status outside the enumerators, as a C caller may pass, is checked
    // through ctypes on the real library by the CPU suite)
    CHECK(qsa_abi_version() == QSA_ABI_VERSION, "abi version");

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi host checks passed\n");
    return 0;
}
