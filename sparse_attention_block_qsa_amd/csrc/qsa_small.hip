// qsa_small.hip -- the QSA block scorer for few query rows (latency-bound
// shapes such as 256 queries against a 128K-token context).
//
// score(g, t, b) = sum_h relu( sum_i k[g, b, i] * q[t, g, h, i] )
// (Strata pull request #228, part 1, score formula.)
//
// Design (gfx950, wave64, v_mfma_f32_32x32x16_f16):
//  * One MFMA row block holds every head of a small query group: its 32 A
//    rows are QPG queries x 2*NP heads (QPG = 16/NP: 4 queries x 8 heads at
//    H = 8, 8 x 4 at H <= 4, 2 x 16 at H > 8).  A row R = 8j + 4*half + i
//    carries query q and head 2p + half for c = 4j + i = p*QPG + q, which
//    is also the output register of that (query, head pair) in the 32x32
//    accumulator, the half (lanes 0-31 / 32-63) picking the head of the
//    pair.  A wave's whole A operand is KS fragments (32 VGPRs at D = 128).
//  * The workgroup's waves own four query groups and walk the same segment
//    of the block axis: 32-block K tiles are staged once through LDS in
//    fragment order (coalesced loads), double-buffered, and read by every
//    wave.  With four waves each owns one query group and scores every tile
//    of a staged chunk (one or two tiles); with eight, waves w and w + 4 own
//    the same query group and split each chunk's tiles (the first half, then
//    the second): a wave's serial work halves and two waves share each SIMD,
//    so one's loads and epilogue overlap the other's.  fp32 queries of many
//    rows go through LDS in fragment order as well, loaded coalesced.
//  * Epilogue per tile: relu per head; v_permlane32_swap of the registers of
//    queries q and q+1 brings the two heads of each pair into one lane; the
//    pair sums are added in ascending pair order.  That is the head-sum
//    order of the wide scorer, so both produce the same bits.
//  * With fp32 queries (the select phase) the chunks are converted on
//    load with the rounding of the conversion kernel, and the first segment
//    of each query group writes the converted rows to the caller's fp16
//    buffer when there is one: the phase needs no conversion launch.  With
//    no full block (a tail only) this kernel serves any number of rows.
//  * The partial last block (n_kv mod bs != 0) is scored by the last segment
//    in the fixed fma order of the tail model, one lane per (query, head);
//    when there are full blocks that segment is one of its own, with no
//    tiles, so that the chain runs beside the tiles.
#include "qsa_internal.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// K tiles staged per barrier and wave half (CH = 1 or 2, 8 or 16 KiB at D =
// 128), double-buffered: at 8 MFMAs per tile, one tile's work is far shorter
// than a load's latency.  With eight waves a chunk is 2*CH tiles (a chunk
// over a shorter remainder stages tiles that are not scored).  Interleaved
// medians of the phase scorer at nq = 256, eight waves: 8 tiles per segment
// (256K keys) 6.49 us with CH = 2, 6.81 us with 1; 4 tiles (128K keys) 4.88
// and 4.84 us.

struct SmallArgs {
    const uint16_t *q16;   // query source when q32 is null
    const float *q32;      // query source when set, converted on load
    uint16_t *q16w;        // with q32: receives the converted rows, or null
    int64_t qts;
    const uint16_t *kblk;
    int64_t khs;
    float *scores;
    int64_t ld_s;
    int32_t G, nq, H;
    int64_t nf;            // full blocks
    int32_t tail;          // block nf is a partial block
    int32_t n_qgroups;     // groups of four query groups (one per wave)
    int32_t n_segs, tiles_per_seg, n_tiles;
    float tail_add;        // added to the partial block's score when nonzero
};

__device__ __forceinline__ float relu_bits(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int32_t, x), 0));
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

template <int D, int NP, bool SRC32, int CH, bool STAGE, int NW>
__global__ __launch_bounds__(64 * NW) void score_small_kernel(SmallArgs a) {
    constexpr int KS = D / 16;
    constexpr int QPG = 16 / NP;
    constexpr int CHUNKS = D / 8;                  // 16-byte chunks per block row
    constexpr int TILE_U4 = CHUNKS * kTileBlocks;
    constexpr int HALVES = NW / kScoreWaves;       // waves per query group
    constexpr int NT = 64 * NW;                    // threads
    constexpr int CT = HALVES * CH;                // tiles per staged chunk
    constexpr int SLOADS = CT * TILE_U4 / NT;      // staging loads per thread per chunk
    static_assert(NP == 1 || NP == 2 || NP == 4 || NP == 8, "head pairs per row block");
    static_assert(TILE_U4 == 256 || TILE_U4 == 512, "D must be 64 or 128");
    static_assert(NW == 4 || NW == 8, "four query groups, one or two waves each");
    static_assert(CH == 1 || CH == 2, "tiles per staged chunk and wave half");
    static_assert(SLOADS * NT == CT * TILE_U4 && SLOADS >= 1, "whole loads per thread");

    // two chunks of K tiles shared by the waves, the four query groups'
    // fragments, and per query group the relu'd tail chains
    __shared__ uint4 kbuf[2][CT * TILE_U4];
    __shared__ uint4 qfrag[STAGE ? kScoreWaves * KS * 64 : 1];
    __shared__ float red[kScoreWaves][QPG][2 * NP];

    const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    const int seg = static_cast<int>(L % a.n_segs);
    const uint32_t rest = L / a.n_segs;
    const int qg4 = static_cast<int>(rest % a.n_qgroups);   // groups of four query groups
    const int g = static_cast<int>(rest / a.n_qgroups);
    const int wv = threadIdx.x >> 6;
    const int w = wv % kScoreWaves;                          // query group slot
    const int hf = wv / kScoreWaves;                         // tile half
    const int l = threadIdx.x & 63;
    const int qg = qg4 * kScoreWaves + w;                    // this wave's query group

    // ---- A operand: this lane's (query, head) row, channels 16s + 8*(l/32) ..
    const int R = l & 31, kc = l >> 5;
    const int c = 4 * (R >> 3) + (R & 3);
    const int p_in = c / QPG, q_in = c % QPG;
    const int h_in = 2 * p_in + ((R >> 2) & 1);
    const int t_in = qg * QPG + q_in;
    const bool a_ok = t_in < a.nq && h_in < a.H;
    const int64_t a_off = static_cast<int64_t>(a_ok ? t_in : 0) * a.qts +
                          static_cast<int64_t>(g * a.H + (a_ok ? h_in : 0)) * D + 8 * kc;

    const int tb = seg * a.tiles_per_seg;
    const int te = min(a.n_tiles, tb + a.tiles_per_seg);
    const uint16_t *kg = a.kblk + static_cast<int64_t>(g) * a.khs;
    float *sbase = a.scores + static_cast<int64_t>(g) * a.nq * a.ld_s;

    // K staging in chunks of CT tiles, double-buffered: the loads of
    // chunk c+1 are in flight while chunk c is scored, one barrier per chunk.
    // A chunk's LDS index U = threadIdx.x + NT*j is tile-major (U = tile *
    // TILE_U4 + u), and within a tile u is chunk-major (u = chunk*32 + block),
    // the B-fragment order: lane l of K-step s reads u = 64*s + l.  Blocks
    // past nf, and tiles past the segment, feed output columns that are never
    // stored: their indices are clamped.
    const int64_t last = a.nf - 1;
    auto kload = [&](int t0, int j) {
        const int U = static_cast<int>(threadIdx.x) + NT * j;
        const int u = U % TILE_U4;
        const int64_t b = min(static_cast<int64_t>(min(t0 + U / TILE_U4, te - 1)) * kTileBlocks +
                                  (u % kTileBlocks), last);
        return *reinterpret_cast<const uint4 *>(kg + b * D + 8 * (u / kTileBlocks));
    };
    uint4 st[SLOADS];
    auto fetch = [&](int t0) {
        #pragma unroll
        for (int j = 0; j < SLOADS; ++j) st[j] = kload(t0, j);
    };
    auto publish = [&](int buf) {
        #pragma unroll
        for (int j = 0; j < SLOADS; ++j) kbuf[buf][threadIdx.x + NT * j] = st[j];
    };
    // the first chunk's loads go out before the queries', so that the two
    // latencies overlap; the tail segment's loads of the partial block's key
    // likewise
    if (tb < te) fetch(tb);   // uniform over the workgroup
    const bool tail_seg = a.tail && seg == a.n_segs - 1;   // uniform
    uint4 kv[KS][2];
    if (tail_seg && hf == 0) {
        const uint16_t *kt = kg + a.nf * D;
        #pragma unroll
        for (int s = 0; s < KS; ++s) {
            kv[s][0] = *reinterpret_cast<const uint4 *>(kt + 16 * s);
            kv[s][1] = *reinterpret_cast<const uint4 *>(kt + 16 * s + 8);
        }
    }

    half8 qa[KS];
    if constexpr (STAGE) {
        // ---- A operand staged through LDS.  The workgroup's
        // 4*QPG query slots x 2*NP head slots x D channels are walked in
        // 8-element chunks, consecutive chunks of a (query, head) row on
        // consecutive threads, so the loads are coalesced: each lane loading
        // its own fragments touches 32 lines per load instruction, and at few
        // rows those requests, not the bytes, set the time.  Each chunk is one
        // lane's fragment of one K-step, converted (f16x8) when the queries
        // are fp32, and written to LDS
        // in fragment order with the lane index XORed by the chunk's index in
        // its row (K-step and half): the 16 chunks of a row land in 16
        // different bank groups, and every wave still reads its A operand
        // conflict-free.  The first segment of each query group also writes
        // the converted rows to the fp16 buffer when there is one.  Chunks of
        // rows past nq and of padded heads are not loaded; their fragments are
        // zeroed when read.
        constexpr int CPR = D / 8;                     // chunks per (query, head) row
        constexpr int MAXJ = 4 * QPG * 2 * NP * CPR / NT;
        static_assert(MAXJ * NT == 4 * QPG * 2 * NP * CPR, "128 rows of chunks over the threads");
        const int t0 = qg4 * kScoreWaves * QPG;
        int64_t off[MAXJ];
        bool ok[MAXJ];
        int dst[MAXJ];
        #pragma unroll
        for (int j = 0; j < MAXJ; ++j) {
            const int ch = static_cast<int>(threadIdx.x) + NT * j;
            const int row = ch / CPR, d8 = ch % CPR;
            const int qs = row / (2 * NP), h = row % (2 * NP);   // query slot, head
            ok[j] = h < a.H && t0 + qs < a.nq;
            off[j] = ok[j] ? static_cast<int64_t>(t0 + qs) * a.qts +
                                 static_cast<int64_t>(g * a.H + h) * D + 8 * d8
                           : 0;
            // fragment slot: wave qs / QPG, K-step d8 / 2, lane of row
            // (query qs % QPG, head h) and half d8 % 2, swizzled by d8
            const int cc = (h >> 1) * QPG + qs % QPG;
            const int ln = 8 * (cc >> 2) + 4 * (h & 1) + (cc & 3) + 32 * (d8 & 1);
            dst[j] = ((qs / QPG) * KS + (d8 >> 1)) * 64 + (ln ^ (d8 & 15));
        }
        uint4 hv[MAXJ];
        if constexpr (SRC32) {
            float4 x0[MAXJ], x1[MAXJ];
            #pragma unroll
            for (int j = 0; j < MAXJ; ++j) {
                x0[j] = *reinterpret_cast<const float4 *>(a.q32 + off[j]);
                x1[j] = *reinterpret_cast<const float4 *>(a.q32 + off[j] + 4);
            }
            #pragma unroll
            for (int j = 0; j < MAXJ; ++j) hv[j] = f16x8(x0[j], x1[j]);
        } else {
            #pragma unroll
            for (int j = 0; j < MAXJ; ++j) hv[j] = *reinterpret_cast<const uint4 *>(a.q16 + off[j]);
        }
        if (SRC32 && a.q16w && seg == 0) {
            #pragma unroll
            for (int j = 0; j < MAXJ; ++j)
                if (ok[j]) *reinterpret_cast<uint4 *>(a.q16w + off[j]) = hv[j];
        }
        #pragma unroll
        for (int j = 0; j < MAXJ; ++j)
            if (ok[j]) qfrag[dst[j]] = hv[j];
        if (tb < te) publish(0);   // uniform over the workgroup
        __syncthreads();
        #pragma unroll
        for (int s = 0; s < KS; ++s)   // chunk index within the row: 2s + l/32
            qa[s] = a_ok ? __builtin_bit_cast(half8, qfrag[(w * KS + s) * 64 + (l ^ ((2 * s + kc) & 15))])
                         : half8{};
    } else {
        // ---- A operand loaded per lane (fp16 queries, or few rows such as
        // one decode query per KV head, where staging would only add its LDS
        // round trip).  All KS fragments' loads are in flight together; fp32
        // queries are converted once they have landed, and the first segment
        // writes the fp16 buffer if any.
        if constexpr (SRC32) {
            float4 x0[KS], x1[KS];
            #pragma unroll
            for (int s = 0; s < KS; ++s) {
                x0[s] = *reinterpret_cast<const float4 *>(a.q32 + a_off + 16 * s);
                x1[s] = *reinterpret_cast<const float4 *>(a.q32 + a_off + 16 * s + 4);
            }
            uint4 hv[KS];
            #pragma unroll
            for (int s = 0; s < KS; ++s) hv[s] = f16x8(x0[s], x1[s]);
            #pragma unroll
            for (int s = 0; s < KS; ++s) qa[s] = a_ok ? __builtin_bit_cast(half8, hv[s]) : half8{};
            if (a.q16w && seg == 0 && hf == 0 && a_ok) {
                #pragma unroll
                for (int s = 0; s < KS; ++s) *reinterpret_cast<uint4 *>(a.q16w + a_off + 16 * s) = hv[s];
            }
        } else {
            #pragma unroll
            for (int s = 0; s < KS; ++s) {
                const half8 v = *reinterpret_cast<const half8 *>(a.q16 + a_off + 16 * s);
                qa[s] = a_ok ? v : half8{};
            }
        }
        if (tb < te) publish(0);   // uniform over the workgroup
        __syncthreads();
    }

    if (tb < te) {   // uniform over the workgroup
        int buf = 0;
        for (int t0 = tb; t0 < te; t0 += CT) {
            const bool more = t0 + CT < te;   // uniform
            if (more) fetch(t0 + CT);
            for (int i = hf * CH; i < hf * CH + CH && t0 + i < te; ++i) {   // uniform per wave
                const int tile = t0 + i;
                const uint4 *kcur = &kbuf[buf][i * TILE_U4 + l];
                floatx16 acc = {};
                #pragma unroll
                for (int s = 0; s < KS; ++s)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        qa[s], __builtin_bit_cast(half8, kcur[64 * s]), s == 0 ? floatx16{} : acc, 0,
                        0, 0);

                // relu per head, then the two heads of each pair into one
                // lane: for queries q, q+1 of pair p (registers r, r+1) the
                // swap gives lanes 0-31 both heads of q and lanes 32-63 both
                // heads of q+1; pair sums are added in ascending pair order
                float pr[16];
                #pragma unroll
                for (int r = 0; r < 16; ++r) pr[r] = relu_bits(acc[r]);
                float tot[QPG / 2];
                #pragma unroll
                for (int p = 0; p < NP; ++p) {
                    #pragma unroll
                    for (int m = 0; m < QPG / 2; ++m) {
                        const int r = p * QPG + 2 * m;
                        const auto sw = __builtin_amdgcn_permlane32_swap(
                            __builtin_bit_cast(uint32_t, pr[r]),
                            __builtin_bit_cast(uint32_t, pr[r + 1]), false, false);
                        const float pair = __builtin_bit_cast(float, static_cast<uint32_t>(sw[0])) +
                                           __builtin_bit_cast(float, static_cast<uint32_t>(sw[1]));
                        tot[m] = p == 0 ? pair : tot[m] + pair;
                    }
                }
                const int64_t b = static_cast<int64_t>(tile) * kTileBlocks + (l & 31);
                #pragma unroll
                for (int m = 0; m < QPG / 2; ++m) {
                    const int t = qg * QPG + 2 * m + kc;
                    if (t < a.nq && b < a.nf) sbase[static_cast<int64_t>(t) * a.ld_s + b] = tot[m];
                }
            }
            if (more) {
                publish(buf ^ 1);
                __syncthreads();
                buf ^= 1;
            }
        }
    }

    // ---- the partial block nf: last segment, one lane per (query, head) chain
    // Lane l < 32 runs the chain of its A row R = l from the query fragments
    // already in registers: v_permlane32_swap gives it the other half of
    // every 16-channel run (held by lane l + 32), so it walks channels
    // 16s .. 16s + 15 in ascending order.
    // With eight waves the first half runs the chains; the second only joins
    // the barrier.
    if (tail_seg) {   // uniform over the workgroup
      if (hf == 0) {
        float acc = 0.0f;
        #pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 x = __builtin_bit_cast(uint4, qa[s]);
            const auto w0 = __builtin_amdgcn_permlane32_swap(x.x, x.x, false, false);
            const auto w1 = __builtin_amdgcn_permlane32_swap(x.y, x.y, false, false);
            const auto w2 = __builtin_amdgcn_permlane32_swap(x.z, x.z, false, false);
            const auto w3 = __builtin_amdgcn_permlane32_swap(x.w, x.w, false, false);
            // lanes 0-31: [0] is the lane's own half (channels 16s .. +7),
            // [1] the half of lane l + 32 (channels 16s + 8 .. +15)
            const uint32_t qw[8] = {w0[0], w1[0], w2[0], w3[0], w0[1], w1[1], w2[1], w3[1]};
            const uint32_t kw[8] = {kv[s][0].x, kv[s][0].y, kv[s][0].z, kv[s][0].w,
                                    kv[s][1].x, kv[s][1].y, kv[s][1].z, kv[s][1].w};
            #pragma unroll
            for (int e = 0; e < 8; ++e) {
                acc = __builtin_fmaf(h2f(kw[e] & 0xffffu), h2f(qw[e] & 0xffffu), acc);
                acc = __builtin_fmaf(h2f(kw[e] >> 16), h2f(qw[e] >> 16), acc);
            }
        }
        const float r = (l < 32 && a_ok && acc > 0.0f) ? acc : 0.0f;
        if (l < 32) red[w][q_in][h_in] = r;   // padded heads and rows hold +0
      }
        __syncthreads();
        if (hf == 0 && l < QPG) {
            const int t = qg * QPG + l;
            if (t < a.nq) {
                float sum = 0.0f;
                for (int h = 0; h < a.H; ++h) sum = sum + red[w][l][h];
                if (a.tail_add != 0.0f) sum = sum + a.tail_add;   // forced-tail rule
                sbase[static_cast<int64_t>(t) * a.ld_s + a.nf] = sum;
            }
        }
    }
}

typedef void (*small_fn)(SmallArgs);

template <int D, bool SRC32, int CH, bool STAGE, int NW>
small_fn pick_np(int np) {
    switch (np) {
        case 1: return score_small_kernel<D, 1, SRC32, CH, STAGE, NW>;
        case 2: return score_small_kernel<D, 2, SRC32, CH, STAGE, NW>;
        case 4: return score_small_kernel<D, 4, SRC32, CH, STAGE, NW>;
        case 8: return score_small_kernel<D, 8, SRC32, CH, STAGE, NW>;
    }
    return nullptr;
}

// src: 0 fp16 queries loaded per lane, 1 fp32 loaded per lane, 2 fp32 staged
// through LDS, 3 fp16 staged through LDS.  Eight waves serve only staged
// queries, and fp16 queries are staged only with eight.
template <int D, int CH, int NW>
small_fn pick_src(int np, int src) {
    if constexpr (NW == 8) {
        if (src == 3) return pick_np<D, false, CH, true, 8>(np);
        if (src == 2) return pick_np<D, true, CH, true, 8>(np);
    } else {
        if (src == 2) return pick_np<D, true, CH, true, 4>(np);
        if (src == 1) return pick_np<D, true, CH, false, 4>(np);
        if (src == 0) return pick_np<D, false, CH, false, 4>(np);
    }
    return nullptr;
}

template <int D>
small_fn pick_ch(int np, int src, int ch, int nw) {
    if (nw == 8) return ch == 2 ? pick_src<D, 2, 8>(np, src) : pick_src<D, 1, 8>(np, src);
    return ch == 2 ? pick_src<D, 2, 4>(np, src) : pick_src<D, 1, 4>(np, src);
}

small_fn pick_small(int D, int np, int src, int ch, int nw) {
    if (D == 128) return pick_ch<128>(np, src, ch, nw);
    if (D == 64) return pick_ch<64>(np, src, ch, nw);
    return nullptr;
}

// Head pairs per MFMA row block: the smallest of 1, 2, 4, 8 that holds H.
int small_pairs(int H) {
    const int np = (H + 1) / 2;
    return np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : 8;
}

}  // namespace

hipError_t launch_score_small(const ScoreGeom &geo, bool tail, hipStream_t s, const float *q32,
                              uint16_t *q16w) {
    if (geo.nq <= 0 || geo.G <= 0 || (geo.nf <= 0 && !tail)) return hipSuccess;
    const int np = small_pairs(geo.H);
    const int qpg = 16 / np;
    const int64_t n_tiles = (geo.nf + kTileBlocks - 1) / kTileBlocks;
    const int64_t n_qgroups = (geo.nq + qpg - 1) / qpg;
    const int64_t n_qg4 = (n_qgroups + kScoreWaves - 1) / kScoreWaves;   // per workgroup: four
    const int64_t base = static_cast<int64_t>(geo.G) * n_qg4;
    // Segments of the block axis: enough workgroups to reach about one per
    // CU (more cost more query reloads than they overlap), each segment
    // keeping at least one tile.
    int64_t segs = 1;
    const int64_t target = 256;
    if (base < target) segs = (target + base - 1) / base;
    const int64_t max_segs = n_tiles > 0 ? n_tiles : 1;
    if (segs > max_segs) segs = max_segs;
    if (segs < 1) segs = 1;
    const int64_t tps = n_tiles > 0 ? (n_tiles + segs - 1) / segs : 0;
    if (n_tiles > 0) segs = (n_tiles + tps - 1) / tps;
    // The partial last block gets a segment of its own, past the tile
    // segments (its tile range is empty), so that its fixed-order chain runs
    // beside the tiles instead of after the last segment's: the decode step's
    // scorer 5.25 -> 3.9 us.  The last segment scores the tail either way.
    if (tail && n_tiles > 0) segs += 1;
    const int64_t grid = base * segs;
    if (grid > 0x7fffffffLL || n_tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // fp32 queries are staged through LDS when a workgroup can hold a full
    // row group.  Interleaved phase medians at nq = 256: 128K keys 10.8 ->
    // 10.0 us, 4K keys 6.9 -> 6.1 us; with one query per KV head staging
    // only adds its LDS round trip (9.9 -> 10.2 us).  Eight waves when the
    // rows fill the workgroup and a segment holds at least two tiles, so that
    // both wave halves have work: interleaved medians at nq = 256, four ->
    // eight waves, phase scorer 5.45 -> 4.91 us at 128K keys, 4.49 -> 3.88 at
    // 64K, 7.87 -> 6.58 at 256K.  fp16 queries are staged only with eight
    // waves, which share the staging: 5.21 -> 4.78 us at 128K (per-lane loads
    // with four waves -> staged with eight), 4.11 -> 3.79 at 64K, 7.62 ->
    // 6.53 at 256K; with four waves staging them loses (3.44 -> 4.07 us at
    // 32K keys, one tile per segment).  Sixteen waves (four per query group)
    // gained 2-3 % at most, and 512 or 128 workgroups of eight waves lost
    // (5.22 and 6.11 us against 4.90 us at 128K keys).
    const bool rows_fill = geo.nq >= kScoreWaves * qpg;
    const int nw = rows_fill && tps >= 2 ? 8 : 4;
    const int src = q32 == nullptr ? (nw > 4 ? 3 : 0) : rows_fill ? 2 : 1;
    // A staged chunk is CH tiles per wave half: with eight waves CH = 2 when
    // the segment is a whole number of 4-tile chunks; with four, when it
    // holds an even number of at least four tiles (2 tiles per segment, the
    // decode step's shape: 9.9 us with CH = 1, 10.05 us with 2).
    const int ch = nw == 8 ? (tps % 4 == 0 ? 2 : 1) : (tps >= 4 && tps % 2 == 0 ? 2 : 1);
    small_fn fn = pick_small(geo.D, np, src, ch, nw);
    if (!fn) return hipErrorInvalidValue;
    SmallArgs a{geo.q16, q32, q32 ? q16w : nullptr, geo.qts, geo.kblk, geo.khs, geo.scores,
                geo.ld_s, geo.G, geo.nq, geo.H, geo.nf, tail ? 1 : 0,
                static_cast<int32_t>(n_qg4), static_cast<int32_t>(segs),
                static_cast<int32_t>(tps), static_cast<int32_t>(n_tiles), geo.tail_add};
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * nw), args, 0, s);
}

}  // namespace qsa
