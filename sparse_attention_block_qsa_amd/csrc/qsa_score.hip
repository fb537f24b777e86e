// qsa_score.hip -- the full-block QSA scorer on CDNA4 MFMA.
//
// score(g, t, b) = sum_h relu( sum_i k[g, b, i] * q[t, g, h, i] )   (b < nf)
// (Strata pull request #228, part 1, score formula; the pages' own kernel is
// an RDNA3 rocWMMA 16x16x16 loop over 8 K-slices, which this does not follow.)
//
// Design (gfx950, wave64, v_mfma_f32_32x32x16_f16):
//  * One wave owns 16 queries of one KV head for a range of block tiles.  Its
//    MFMA A operand is 32 rows = (2 heads) x (16 queries): lane l holds
//    q[t0 + l%16][g][2p + (l%32)/16][16s + 8*(l/32) .. +7] for head pair p
//    and K-step s.  All of the wave's query rows (H*D fp16 per query, 128
//    VGPRs at H*D = 1024) stay in registers for the whole kernel: queries are
//    the operand with 8x the reuse, so they are the stationary one.
//  * The B operand is 32 blocks of K_blk, N = block axis: lane l holds
//    k[b0 + l%32][16s + 8*(l/32) .. +7].  A 32-block tile (8 KiB at D=128) is
//    staged once per workgroup in LDS, stored in fragment order so that
//    every ds_read_b128 is lane-contiguous, and reused by the four waves and
//    by every head pair.
//  * The 32x32 accumulator of one head pair holds, per lane, the same
//    (query, block) cells for both heads (registers r and r+8), so the relu
//    and the head sum are lane-local: pair = relu(acc[u]) + relu(acc[u+8]),
//    then tot[u] += pair, pairs ascending.  Two waves per SIMD (<= 256 VGPRs
//    each) let one wave's relu/add epilogue run on the VALU while the matrix
//    core works on the other wave's MFMAs.
//  * Stores: for a fixed accumulator register the 64 lanes hold 2 query rows
//    x 32 consecutive blocks, i.e. two full 128-byte row segments; they are
//    raw buffer stores, so masked lanes cost no branch.
//  * K tiles go through an LDS ring with one barrier per tile; the LDS reads
//    are pinned one K-step ahead of the MFMAs that use them.  Each tile's
//    global loads are issued three tiles ahead (a four-slot ring) where the
//    registers allow it, so that the wait for them, which on this
//    architecture also waits for every store issued before them, does not
//    wait for the previous tile's score stores.
//  * Ragged edges: query rows >= nq load zeros, blocks >= nf repeat block
//    nf-1 (MFMA output columns are independent, and those columns are never
//    stored), and stores are masked, so the write set is exactly
//    scores[g*nq + t][0, nf).
//  * A partial last block (n_kv mod bs != 0) is scored at the end by the
//    last split of each query group, from the same resident query registers,
//    in the fixed fma order of the tail model, so the queries are read from
//    HBM once for all nb blocks.
//  * fp32 queries (the select phase) are read and converted to fp16 bits on
//    load with the conversion kernel's own instruction (f16x8), and the
//    first split of each query group writes those bits to the caller's fp16
//    buffer when there is one: the phase needs no conversion launch and
//    reads the queries from HBM once.
//  * Grid: (KV head, 64-query group, block split), with logical ids laid out
//    so that each XCD (blockIdx % 8) takes a contiguous range: the splits of
//    one query group and the query groups of one KV head share that XCD's L2.
//  * The 16x16x32 form (M16: one head pass with buffer stores, the instances
//    the prefill scorers run).  The same tile on v_mfma_f32_16x16x32_f16:
//    A row tiles of 4 queries x 4 heads (lane l holds row l%16 = 4*query +
//    head of its quad, channels 32s + 8*(l/16) .. +7), B column tiles of 16
//    blocks read from the same LDS ring (chunk 4s + l/16, block 16c + l%16),
//    and each lane's four accumulator rows are four heads of one query, so
//    the relu and the head sum stay lane-local, in the same order.  A D = 128
//    dot product chained over four 16x16x32 steps has the bits of the eight
//    32x32x16 steps (a probe over 20,480 dot products, cancellation
//    included, found no difference), so both forms, the small and the decode
//    scorer agree bit for bit.  Under the chip's power limit a loop of the
//    16x16x32 instruction sustains more than one of the 32x32x16 (measured
//    beside the scorers by the benchmark), and at the prefill chunk the
//    fp16-input scorer went 227 -> 213 us (fp32 queries 254 -> 252 us).
//    After the epilogue, one v_permlane16_swap per register pair turns the
//    two 16-block column tiles of a query quad into 32-block rows, so the
//    stores write whole 128-byte row segments (+1.2 % with 64-byte ones).
//  * Fused selection (SEL > 0, one split per query group): after its last
//    tile and the partial block, each wave selects the top-k of its own 16
//    query rows, whose scores (every block, tail included) only it wrote,
//    with the one-wave row selection of the top-k selector
//    (qsa_topk_row.h), so the phase needs no selector launch.  The scores
//    are still written; the selection re-reads them.
#include "qsa_internal.h"
#include "qsa_stream_row.h"
#include "qsa_topk_row.h"

namespace qsa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct ScoreArgs {
    const uint16_t *q16;   // query source when q32 is null
    const float *q32;      // query source when set, converted on load
    uint16_t *q16w;        // with q32: receives the converted rows, or null
    int64_t qts;
    const uint16_t *kblk;
    int64_t khs;
    float *scores;
    int64_t ld_s;
    int32_t G, nq, H;
    int32_t h0, nh;        // heads [h0, h0 + nh) in this pass
    int32_t accumulate;    // 1: continue the head sum already in scores
    int64_t nf;
    int32_t n_qgroups, n_splits, tiles_per_split, n_tiles;
    float tail_add;        // added to the partial block's score when nonzero
                           // (last head pass only)
    // fused selection (SEL > 0): ids / vals of row g*nq + t go to
    // ids[(g*dst_group_rows + dst_row0 + t)*ld_ids + 0 .. k)
    int32_t *ids;
    int64_t ld_ids;
    float *vals;
    int32_t k, nb;
    int64_t dst_group_rows, dst_row0;
};

// s_waitcnt immediate for vmcnt(0) with the other counters left free
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kVmcnt0 = 0x0F70;

// Cache policy of the score stores: non-temporal.  The scores are written
// once and read back by the selector long after they would have left the
// caches, so they stream to memory without displacing the queries and keys.
constexpr int kStoreNT = 2;

// relu on fp32 bits: as signed integers, negative floats (and -0) are < 0 and
// non-negative floats keep their order, so max(bits, 0) is relu(x) with -0
// mapped to +0.  One v_max_i32, no NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int32_t, x), 0));
}

template <int D, int NP, bool ACCUM, bool BUF, bool TAIL, bool SRC32, int SEL = 0,
          bool STREAM = false, bool M16 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_full_kernel(ScoreArgs a) {
    constexpr int KS = D / 16;              // MFMA K-steps per head
    // M16: the same tile on v_mfma_f32_16x16x32_f16 (row tiles of 4 queries
    // x 4 heads, two 16-block column tiles); see the design notes above
    constexpr int KS16 = D / 32;            // its K-steps
    constexpr int NHH = (2 * NP + 3) / 4;   // head quads in the pass
    constexpr int RT = 4 * NHH;             // row tiles: 4 query quads x NHH
    static_assert(!M16 || (!ACCUM && BUF && SEL == 0 && !STREAM),
                  "the 16x16x32 form: one head pass, buffer stores, no selection");
    constexpr int CHUNKS = D / 8;           // 16-byte chunks per block row
    constexpr int TILE_U4 = CHUNKS * kTileBlocks;
    constexpr int LOADS = TILE_U4 / 256;    // uint4 per thread per tile
    static_assert(TILE_U4 % 256 == 0 && (LOADS == 1 || LOADS == 2), "D must be 64 or 128");
    static_assert(NP >= 1 && NP <= 4, "at most four head pairs per pass");

    // Ring of K tiles: while tile t is consumed, tile t+1 is already
    // published (so its first fragments can be read before the barrier) and
    // tile t+2 is being staged.  Tile t+2's global loads were issued DIST
    // tiles ahead of their use: with DIST = 3 they were issued one tile
    // earlier and held in registers, so the vector-memory wait before they
    // are written to LDS (the counter covers loads and stores in issue
    // order) no longer waits for the score stores of tile t-1.  Prefill
    // chunk, interleaved medians: fp16 queries 243 -> 227 us, fp32 queries
    // 267 -> 253 us.  It costs 8 registers, which the accumulating pass and
    // the 64-bit store path do not have to spare (they would spill).
    // The streaming selection keeps DIST = 2: its candidate buffers need the
    // LDS of the fourth ring slot, and its state the registers.
    constexpr int DIST = (!ACCUM && BUF && !STREAM) ? 3 : 2;
    constexpr int NS = DIST + 1;   // ring slots
    __shared__ uint4 kbuf[NS][TILE_U4];
    __shared__ uint4 ktail[TAIL ? CHUNKS : 1];   // the partial block's key
    // fused selection: per wave 128 candidate composites and the row's values
    __shared__ uint64_t sel_slot[SEL > 0 ? kScoreWaves : 1][SEL > 0 ? 128 : 1];
    __shared__ uint32_t sel_stash[SEL > 0 ? kScoreWaves : 1][SEL > 0 ? 64 * SEL : 1];
    static_assert(SEL == 0 || (!ACCUM && BUF), "fused selection: one head pass, buffer stores");
    // streaming selection: per wave and score row a buffer of kStreamCap
    // candidates (score bits, block id) in block-id order
    // (each wave's region ends with one dummy slot per lane)
    constexpr int kStreamWave = kWaveQueries * kStreamCap + 64;
    __shared__ uint32_t st_val[STREAM ? kScoreWaves * kStreamWave : 1];
    __shared__ uint16_t st_id[STREAM ? kScoreWaves * kStreamWave : 1];
    __shared__ __attribute__((aligned(16))) float st_thr[kScoreWaves][STREAM ? kWaveQueries : 4];
    __shared__ uint32_t st_kb[kScoreWaves][STREAM ? kWaveQueries : 1];
    static_assert(!STREAM || (!ACCUM && SEL == 0), "streaming selection: one head pass");

    const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    const int split = static_cast<int>(L % a.n_splits);
    const uint32_t rest = L / a.n_splits;
    const int qg = static_cast<int>(rest % a.n_qgroups);
    const int g = static_cast<int>(rest / a.n_qgroups);

    const int tb = split * a.tiles_per_split;
    const int te = min(a.n_tiles, tb + a.tiles_per_split);
    if (tb >= te) return;   // uniform over the workgroup

    const int w = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int t_base = qg * kGroupQueries + w * kWaveQueries;

    // ---- K tile staging ----------------------------------------------------
    // LDS index u = threadIdx.x + 256*c is chunk-major (u = chunk*32 + block),
    // which is also the MFMA B-fragment order: lane l of K-step s reads
    // u = 64*s + l, lane-contiguous.  Blocks past nf (and tiles past the
    // split) only feed MFMA output columns that are never stored, so their
    // rows may be any in-bounds data: the indices are clamped.
    const uint16_t *kg = a.kblk + static_cast<int64_t>(g) * a.khs;
    const int u0 = threadIdx.x, u1 = threadIdx.x + 256;
    const int off0 = 8 * (u0 / kTileBlocks), off1 = 8 * (u1 / kTileBlocks);
    const int bb0 = u0 % kTileBlocks, bb1 = u1 % kTileBlocks;
    const int64_t last = a.nf - 1;
    auto kload = [&](int tile, int bb, int off) {
        const int64_t b = min(static_cast<int64_t>(min(tile, te - 1)) * kTileBlocks + bb, last);
        return *reinterpret_cast<const uint4 *>(kg + b * D + off);
    };

    // prologue loads: tiles tb and tb+1 (and the tail key), published below
    uint4 x0 = kload(tb, bb0, off0), y0 = kload(tb + 1, bb0, off0);
    uint4 x1 = make_uint4(0, 0, 0, 0), y1 = make_uint4(0, 0, 0, 0);
    if constexpr (LOADS == 2) {
        x1 = kload(tb, bb1, off1);
        y1 = kload(tb + 1, bb1, off1);
    }
    // DIST = 3: tile tb+2's loads, written to LDS in the first iteration
    uint4 p0 = make_uint4(0, 0, 0, 0), p1 = make_uint4(0, 0, 0, 0);
    if constexpr (DIST == 3) {
        p0 = kload(tb + 2, bb0, off0);
        if constexpr (LOADS == 2) p1 = kload(tb + 2, bb1, off1);
    }
    uint4 kt = make_uint4(0, 0, 0, 0);
    const bool tail_wg = TAIL && split == a.n_splits - 1;   // uniform
    if (tail_wg && threadIdx.x < CHUNKS)
        kt = reinterpret_cast<const uint4 *>(kg + a.nf * D)[threadIdx.x];

    // ---- stationary query fragments --------------------------------------
    // Issued after the first K tiles' loads and in K-step order, so that the
    // K tiles are published while the queries are still in flight and the
    // first MFMAs wait only for the fragments of their own K-step.  Every
    // lane loads from an in-bounds address, without branches.  Rows of
    // queries past nq read query 0: they only feed MFMA rows that are never
    // stored.  A head past the pass (only the second head of the last pair,
    // when nh is odd) is zeroed, since it would enter the head sum.  fp32
    // queries (SRC32) are converted on load; the first split of each query
    // group writes their fp16 bits for the real rows and heads, so every
    // element of the workspace is written exactly once.
    half8 qa[M16 ? 1 : NP][M16 ? 1 : KS];
    half8 qa16[M16 ? RT : 1][M16 ? KS16 : 1];
    const int hh = (l >> 4) & 1;   // this lane's head within a pair
    // This lane's row of head hh in the workspace, channel 8*(l/32) (head
    // 2p + hh is 2p*D further on), or null when it writes nothing: the first
    // split of each query group writes the real rows.
    uint16_t *qw = nullptr;
    if constexpr (!M16) {
        {
            const int tq = l & 15, kc = l >> 5;
            const int t = t_base + tq;
            const int64_t trow = static_cast<int64_t>(t < a.nq ? t : 0) * a.qts;
            int64_t qoff[NP];
            #pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int h = 2 * p + hh;
                qoff[p] = trow + static_cast<int64_t>(g * a.H + a.h0 + (h < a.nh ? h : 0)) * D + 8 * kc;
            }
            if (SRC32 && a.q16w != nullptr && split == 0 && t < a.nq && hh < a.nh)
                qw = a.q16w + qoff[0];
            if constexpr (!SRC32) {
                #pragma unroll
                for (int s = 0; s < KS; ++s) {
                    #pragma unroll
                    for (int p = 0; p < NP; ++p)
                        qa[p][s] = *reinterpret_cast<const half8 *>(a.q16 + qoff[p] + 16 * s);
                }
            } else {
                // fp32 fragments (8 VGPRs each, twice the fp16 size) in batches
                // of kQBatch, kQDepth batches in flight: each batch is converted
                // as it lands and the registers it frees take the next batch's
                // loads.  Left free, the compiler hoists every load above the
                // conversions and runs out of registers.
                constexpr int F = KS * NP;                    // fragments, K-step major
                // (the accumulating pass with 64-bit store addressing holds more
                // registers: one batch fewer in flight)
                constexpr int kQBatch = 4, kQDepth = 3;
                constexpr int NBAT = (F + kQBatch - 1) / kQBatch;
                float4 x0[F], x1[F];
                auto issue = [&](int b) {
                    #pragma unroll
                    for (int j = 0; j < kQBatch; ++j) {
                        const int f = b * kQBatch + j;
                        if (f < F) {
                            const float *src = a.q32 + qoff[f % NP] + 16 * (f / NP);
                            x0[f] = *reinterpret_cast<const float4 *>(src);
                            x1[f] = *reinterpret_cast<const float4 *>(src + 4);
                        }
                    }
                };
                #pragma unroll
                for (int b = 0; b < kQDepth && b < NBAT; ++b) issue(b);
                #pragma unroll
                for (int b = 0; b < NBAT; ++b) {
                    #pragma unroll
                    for (int j = 0; j < kQBatch; ++j) {
                        const int f = b * kQBatch + j;
                        if (f < F) {
                            const uint4 h = f16x8(x0[f], x1[f]);
                            qa[f % NP][f / NP] = __builtin_bit_cast(half8, h);
                            // an empty statement that uses the converted fragment
                            // and orders memory: the conversion stays before the
                            // next batch's loads, which cannot move above it
                            asm volatile("" ::"v"(h.x), "v"(h.y), "v"(h.z), "v"(h.w) : "memory");
                        }
                    }
                    if (b + kQDepth < NBAT) issue(b + kQDepth);
                }
            }
            if (2 * NP > a.nh) {   // uniform
                #pragma unroll
                for (int s = 0; s < KS; ++s)
                    if (hh) qa[NP - 1][s] = half8{};
            }
        }
    } else {
        // 16x16x32 A fragments: row tile i = (query quad i / NHH, head quad
        // i % NHH); lane l holds row l%16 = 4*(query in quad) + head in quad,
        // channels 32s + 8*(l/16) .. +7 of K-step s.  Rows past nq read query
        // 0 (never stored); heads past the pass are zeroed below.
        const int m = l & 15, kc = l >> 4;
        const int qq = m >> 2, hq = m & 3;
        int64_t qoff[RT];
        #pragma unroll
        for (int i = 0; i < RT; ++i) {
            const int t = t_base + 4 * (i / NHH) + qq;
            const int h = 4 * (i % NHH) + hq;
            qoff[i] = static_cast<int64_t>(t < a.nq ? t : 0) * a.qts +
                      static_cast<int64_t>(g * a.H + a.h0 + (h < a.nh ? h : 0)) * D + 8 * kc;
        }
        if constexpr (!SRC32) {
            #pragma unroll
            for (int s = 0; s < KS16; ++s) {
                #pragma unroll
                for (int i = 0; i < RT; ++i)
                    qa16[i][s] = *reinterpret_cast<const half8 *>(a.q16 + qoff[i] + 32 * s);
            }
        } else {
            // batched as above: each batch converted as it lands
            constexpr int F = KS16 * RT;                  // fragments, K-step major
            constexpr int kQBatch = 4, kQDepth = 3;
            constexpr int NBAT = (F + kQBatch - 1) / kQBatch;
            float4 x0[F], x1[F];
            auto issue = [&](int b) {
                #pragma unroll
                for (int j = 0; j < kQBatch; ++j) {
                    const int f = b * kQBatch + j;
                    if (f < F) {
                        const float *src = a.q32 + qoff[f % RT] + 32 * (f / RT);
                        x0[f] = *reinterpret_cast<const float4 *>(src);
                        x1[f] = *reinterpret_cast<const float4 *>(src + 4);
                    }
                }
            };
            #pragma unroll
            for (int b = 0; b < kQDepth && b < NBAT; ++b) issue(b);
            #pragma unroll
            for (int b = 0; b < NBAT; ++b) {
                #pragma unroll
                for (int j = 0; j < kQBatch; ++j) {
                    const int f = b * kQBatch + j;
                    if (f < F) {
                        const uint4 h = f16x8(x0[f], x1[f]);
                        qa16[f % RT][f / RT] = __builtin_bit_cast(half8, h);
                        asm volatile("" ::"v"(h.x), "v"(h.y), "v"(h.z), "v"(h.w) : "memory");
                    }
                }
                if (b + kQDepth < NBAT) issue(b + kQDepth);
            }
            // the real rows and heads into the fp16 workspace, after the
            // last load (first split of each query group)
            if (a.q16w != nullptr && split == 0) {
                #pragma unroll
                for (int i = 0; i < RT; ++i) {
                    const int t = t_base + 4 * (i / NHH) + qq;
                    const int h = 4 * (i % NHH) + hq;
                    if (t < a.nq && h < a.nh) {
                        #pragma unroll
                        for (int s = 0; s < KS16; ++s)
                            *reinterpret_cast<uint4 *>(a.q16w + qoff[i] + 32 * s) =
                                __builtin_bit_cast(uint4, qa16[i][s]);
                    }
                }
            }
        }
        // heads past the pass would enter the head sum (odd nh): zero rows
        if (4 * NHH > a.nh) {   // uniform
            #pragma unroll
            for (int i = 0; i < RT; ++i) {
                if (4 * (i % NHH) + hq >= a.nh) {
                    #pragma unroll
                    for (int s = 0; s < KS16; ++s) qa16[i][s] = half8{};
                }
            }
        }
    }

    // The converted queries into the fp16 workspace (SRC32, when the caller
    // gave one), after the last query load: the workspace may alias the fp32
    // queries as far as the compiler knows, so a store between the loads
    // would hold back every load after it.  Temporal stores: the 32-byte
    // pieces of each line merge in L2.
    if constexpr (SRC32 && !M16) {
        if (qw != nullptr) {
            #pragma unroll
            for (int s = 0; s < KS; ++s) {
                #pragma unroll
                for (int p = 0; p < NP; ++p)
                    if (2 * p + hh < a.nh)
                        *reinterpret_cast<uint4 *>(qw + 2 * p * D + 16 * s) = __builtin_bit_cast(uint4, qa[p][s]);
            }
        }
    }

    // ---- output addressing -------------------------------------------------
    // Lane l holds, for register u (0..7), query t_base + 8*(u/4) + 4*(l/32)
    // + u%4 and block tile*32 + l%32 (M16, after the epilogue's lane swap:
    // query t_base + 4*(u/2) + u%2 + 2*(l/32) and the same block).  With BUF the stores are raw buffer
    // stores over this KV head's rows: an offset >= 2^30 (past the region,
    // which the host limits to 2^30 bytes) is dropped by the hardware, so
    // masked lanes need no branch.
    float *srow_base = a.scores + static_cast<int64_t>(g) * a.nq * a.ld_s;
    const int bl = l & 31;
    // BUF: byte offsets (the region is below 2^30 bytes, so they fit 32
    // bits and kOut marks a masked row); otherwise element offsets and -1.
    constexpr uint32_t kOut = 0x40000000u;
    uint32_t rowoff[8];
    int64_t rowel[8];
    #pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int t = M16 ? t_base + 4 * (u >> 1) + (u & 1) + 2 * (l >> 5)
                          : t_base + 8 * (u >> 2) + 4 * (l >> 5) + (u & 3);
        if constexpr (BUF)
            rowoff[u] = t < a.nq ? static_cast<uint32_t>(static_cast<int64_t>(t) * a.ld_s * 4) : kOut;
        else
            rowel[u] = t < a.nq ? static_cast<int64_t>(t) * a.ld_s : -1;
    }
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        srow_base, 0, BUF ? static_cast<int>(static_cast<int64_t>(a.nq) * a.ld_s * 4) : 0,
        0x00020000 /* 32-bit elements, raw */);

    // prologue: tiles tb and tb+1 into slots 0 and 1 (and the tail key)
    {
        if (tail_wg && threadIdx.x < CHUNKS) ktail[threadIdx.x] = kt;
        kbuf[0][u0] = x0;
        kbuf[1][u0] = y0;
        if constexpr (LOADS == 2) {
            kbuf[0][u1] = x1;
            kbuf[1][u1] = y1;
        }
    }
    __syncthreads();
    // Every query fragment (and the prologue's K loads) has landed before the
    // tile loop.  Without this wait the compiler's wait counting carries the
    // query loads into the loop as possibly outstanding, and, because the
    // vector-memory counter also counts stores in issue order, the waits it
    // then places before the MFMAs of every tile (vmcnt(33) down to vmcnt(2))
    // wait for the previous tile's score stores to be acknowledged.
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    int slot = 0;   // ring slot of the current tile

    // ---- streaming selection state (STREAM) -------------------------------
    // Row r of the wave is query t_base + r; in a tile, register u holds row
    // 8*(u/4) + (u%4) in lanes 0-31 and that row + 4 in lanes 32-63.  Per
    // row: the candidate count (uniform, in scalar registers), and in LDS its
    // admission threshold (st_thr) and a key no later number is below
    // (st_kb), both written only when the row is compacted.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint32_t *wval = st_val + wu * kStreamWave;
    uint16_t *wid = st_id + wu * kStreamWave;
    const uint32_t dummy = kWaveQueries * kStreamCap + l;   // this lane's dummy slot
    float *wthr = st_thr[wu];
    uint32_t *wkb = st_kb[wu];
    const bool upper = l >= 32;
    const int kk = static_cast<int>(min(static_cast<int64_t>(a.k), static_cast<int64_t>(a.nb)));
    int cnt[kWaveQueries];
    #pragma unroll
    for (int r = 0; r < kWaveQueries; ++r) cnt[r] = 0;
    if constexpr (STREAM) {
        if (l < kWaveQueries) {
            wthr[l] = -__builtin_inff();
            wkb[l] = 0;
        }
        wave_lds_sync();
    }
    // Compacts the rows in need (and the rows within 40 of full, so that
    // rows filling together are compacted in one pass).
    auto stream_compact_rows = [&](uint32_t need) __attribute__((always_inline)) {
        #pragma unroll
        for (int r = 0; r < kWaveQueries; ++r)
            if (cnt[r] > kStreamCap - 40) need |= 1u << r;
        uint32_t cv = 0;
        #pragma unroll
        for (int r = 0; r < kWaveQueries; ++r) cv = lane_set(cv, l, r, cnt[r]);
        need = uni(need);
        while (need) {
            const int r = uni(__builtin_ctz(need));
            need &= need - 1;
            uint32_t adm, kb;
            const int n = stream_compact(wval + r * kStreamCap, wid + r * kStreamCap,
                                         uni(__builtin_amdgcn_readlane(cv, r)), kk, l, &adm, &kb);
            cv = lane_set(cv, l, r, n);
            if (l == 0) {
                wthr[r] = stream_admit_floor(adm);
                wkb[r] = kb;
            }
        }
        #pragma unroll
        for (int r = 0; r < kWaveQueries; ++r) cnt[r] = uni(__builtin_amdgcn_readlane(cv, r));
        wave_lds_sync();
    };
    // This lane's rows' thresholds (rows 4h .. 4h+3 and 8+4h .. 8+4h+3 for
    // registers 0-3 and 4-7), held in registers and reloaded after each
    // compaction.
    float tv[8];
    auto load_tv = [&]() __attribute__((always_inline)) {
        const float4 t0 = *reinterpret_cast<const float4 *>(wthr + (upper ? 4 : 0));
        const float4 t1 = *reinterpret_cast<const float4 *>(wthr + (upper ? 12 : 8));
        tv[0] = t0.x; tv[1] = t0.y; tv[2] = t0.z; tv[3] = t0.w;
        tv[4] = t1.x; tv[5] = t1.y; tv[6] = t1.z; tv[7] = t1.w;
    };
    if constexpr (STREAM) load_tv();
    // One tile's scores (tot, columns tile*32 + l%32) into the row buffers.
    auto stream_tile = [&](int tile, const float (&tot)[8]) __attribute__((always_inline)) {
        const int bcol = tile * kTileBlocks + bl;
        const bool colv = bcol < a.nf;   // columns of real blocks
        const uint64_t colm = ballot_b(colv);
        // rows that would overflow: compacted before anything is appended
        uint32_t need = 0;
        #pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint64_t m = ballot_b(!(tot[u] < tv[u])) & colm;   // NaN passes
            const int rA = 8 * (u >> 2) + (u & 3);
            if (cnt[rA] + __popc(static_cast<uint32_t>(m)) > kStreamCap) need |= 1u << rA;
            if (cnt[rA + 4] + __popc(static_cast<uint32_t>(m >> 32)) > kStreamCap)
                need |= 1u << (rA + 4);
        }
        need = uni(need);
        if (need) {   // uniform; rare once the thresholds have risen
            stream_compact_rows(need);
            load_tv();
        }
        // append: lanes of a row write in lane (block) order after the row's
        // last entry; mbcnt over the 64-lane mask gives the lower half its
        // position directly and the upper half after the lower half's count,
        // which the uniform adjustment removes
        #pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int rA = 8 * (u >> 2) + (u & 3), rB = rA + 4;
            const bool ge = !(tot[u] < tv[u]);
            const uint64_t m = ballot_b(ge) & colm;
            const uint32_t mlo = static_cast<uint32_t>(m), mhi = static_cast<uint32_t>(m >> 32);
            const int nA = __popc(mlo), nB = __popc(mhi);
            const int sb = cnt[rA] + rA * kStreamCap;
            const int adj = cnt[rB] + rB * kStreamCap - nA - sb;
            const uint32_t b = upper ? static_cast<uint32_t>(adj) : 0u;
            uint32_t idx = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, b)) + sb;
            // every lane writes (no branch, so the counts stay scalar): the
            // lanes that do not pass write their own dummy slot.  The empty
            // asm keeps the compiler from turning the select into a branch
            // around the position arithmetic.
            asm volatile("" : "+v"(idx));
            const uint32_t at = (ge && colv) ? idx : dummy;
            wval[at] = __builtin_bit_cast(uint32_t, tot[u]);
            wid[at] = static_cast<uint16_t>(bcol);
            cnt[rA] = uni(cnt[rA] + nA);
            cnt[rB] = uni(cnt[rB] + nB);
        }
    };
    // The tail block's candidate of every row (lane r < 16: row r's score),
    // appended after compacting the rows whose buffer is full.
    auto stream_tail = [&](float sum) __attribute__((always_inline)) {
        uint32_t cv = 0;
        #pragma unroll
        for (int r = 0; r < kWaveQueries; ++r) cv = lane_set(cv, l, r, cnt[r]);
        const bool lr = l < kWaveQueries;
        wave_lds_sync();
        bool tp = lr && !(sum < wthr[l & 15]);
        uint32_t full = uni(static_cast<uint32_t>(ballot_b(tp && cv == static_cast<uint32_t>(kStreamCap))));
        if (full) {   // uniform
            while (full) {
                const int r = uni(__builtin_ctz(full));
                full &= full - 1;
                uint32_t adm, kb;
                const int n = stream_compact(wval + r * kStreamCap, wid + r * kStreamCap, kStreamCap,
                                             kk, l, &adm, &kb);
                cv = lane_set(cv, l, r, n);
                if (l == 0) {
                    wthr[r] = stream_admit_floor(adm);
                    wkb[r] = kb;
                }
            }
            wave_lds_sync();
            tp = lr && !(sum < wthr[l & 15]);
        }
        if (tp) {
            wval[l * kStreamCap + cv] = __builtin_bit_cast(uint32_t, sum);
            wid[l * kStreamCap + cv] = static_cast<uint16_t>(a.nf);
        }
        const uint64_t added = ballot_b(tp);
        #pragma unroll
        for (int r = 0; r < kWaveQueries; ++r)
            cnt[r] = uni(__builtin_amdgcn_readlane(cv, r) + static_cast<int>((added >> r) & 1));
    };

    // This lane's B fragments of a tile's first K-step(s) in the ring: K-steps
    // 0 and 1 (32x32x16), or column tiles 0 and 1 of K-step 0 (M16: chunk
    // 4s + l/16, block 16c + l%16, i.e. +128 per K-step).
    const int fo0 = M16 ? 32 * (l >> 4) + (l & 15) : l;
    const int fo1 = M16 ? fo0 + 16 : 64 + l;
    half8 kf0 = __builtin_bit_cast(half8, kbuf[0][fo0]);
    half8 kf1 = __builtin_bit_cast(half8, kbuf[0][fo1]);

    // One tile: its loads go to ld (tile + DIST), and tile + 2 is staged from
    // pw (DIST = 3: loaded by the previous tile) or from ld (DIST = 2).  The
    // loop below alternates the two register sets, so that no copy of a load
    // in flight (which would wait for it) is needed.
    uint4 q0 = make_uint4(0, 0, 0, 0), q1 = make_uint4(0, 0, 0, 0);
    auto step = [&](int tile, uint4 &pw0, uint4 &pw1, uint4 &ld0, uint4 &ld1) __attribute__((always_inline)) {
        const int nslot = slot + 1 == NS ? 0 : slot + 1;
        const int wslot = nslot + 1 == NS ? 0 : nslot + 1;   // held tile + 2 - NS: free
        ld0 = kload(tile + DIST, bb0, off0);
        if constexpr (LOADS == 2) ld1 = kload(tile + DIST, bb1, off1);

        const int bcol = tile * kTileBlocks + bl;
        const uint32_t coloff = bcol < a.nf ? static_cast<uint32_t>(bcol) * 4 : kOut;

        float tot[8];
        #pragma unroll
        for (int u = 0; u < 8; ++u) {
            tot[u] = 0.0f;
            if constexpr (ACCUM) {
                if constexpr (BUF) {
                    tot[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          rs, static_cast<int>(rowoff[u] + coloff), 0, 0));
                } else if (rowel[u] >= 0 && coloff != kOut) {
                    tot[u] = srow_base[rowel[u] + bcol];
                }
            }
        }

        // MFMA phase: K-step outer so the NP MFMAs sharing a B fragment are
        // independent; fragment s+2 is read from LDS one step ahead of use.
        // The wave raises its issue priority for the phase: of the two waves
        // on a SIMD, the one with MFMAs to issue goes first, and the other
        // runs its epilogue in the gaps (a lasting ping-pong instead of both
        // waves reaching their epilogues together).
        floatx16 acc[M16 ? 1 : NP];
        floatx4 acc16[M16 ? RT : 1][2];
        if constexpr (M16) {
            // every row tile against both column tiles per K-step; the next
            // K-step's two fragments are read from LDS one step ahead
            __builtin_amdgcn_s_setprio(1);
            const uint4 *kcur = &kbuf[slot][0];
            half8 kb0 = kf0, kb1 = kf1;
            #pragma unroll
            for (int s = 0; s < KS16; ++s) {
                half8 nb0 = kb0, nb1 = kb1;
                if (s + 1 < KS16) {
                    nb0 = __builtin_bit_cast(half8, kcur[fo0 + 128 * (s + 1)]);
                    nb1 = __builtin_bit_cast(half8, kcur[fo1 + 128 * (s + 1)]);
                }
                #pragma unroll
                for (int i = 0; i < RT; ++i) {
                    acc16[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        qa16[i][s], kb0, (s == 0) ? floatx4{} : acc16[i][0], 0, 0, 0);
                    acc16[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        qa16[i][s], kb1, (s == 0) ? floatx4{} : acc16[i][1], 0, 0, 0);
                }
                kb0 = nb0;
                kb1 = nb1;
            }
            __builtin_amdgcn_sched_group_barrier(0x020, LOADS, 0);   // staging loads
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // K-step 1's fragments
            #pragma unroll
            for (int s = 0; s < KS16; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * RT, 0);
                if (s + 2 < KS16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_s_setprio(0);
        } else {
            __builtin_amdgcn_s_setprio(1);
            const uint4 *kcur = &kbuf[slot][l];
            half8 kf = kf0, kn = kf1;
            #pragma unroll
            for (int s = 0; s < KS; ++s) {
                half8 k2 = kn;
                if (s + 2 < KS) k2 = __builtin_bit_cast(half8, kcur[64 * (s + 2)]);
                #pragma unroll
                for (int p = 0; p < NP; ++p) {
                    const floatx16 c = (s == 0) ? floatx16{} : acc[p];
                    acc[p] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[p][s], kf, c, 0, 0, 0);
                }
                kf = kn;
                kn = k2;
            }
            // Keep the LDS reads a step ahead of their MFMAs (the scheduler would
            // otherwise sink each read next to its first use).
            __builtin_amdgcn_sched_group_barrier(0x020, LOADS, 0);   // staging loads
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // fragments 2, 3
            #pragma unroll
            for (int s = 0; s < KS; ++s) {
                __builtin_amdgcn_sched_group_barrier(0x008, NP, 0);
                if (s + 4 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }

            __builtin_amdgcn_s_setprio(0);
        }

        // the next tile was published an iteration ago: fetch its first two
        // fragments now, then stage tile+2 into the free slot
        kf0 = __builtin_bit_cast(half8, kbuf[nslot][fo0]);
        kf1 = __builtin_bit_cast(half8, kbuf[nslot][fo1]);
        kbuf[wslot][u0] = DIST == 3 ? pw0 : ld0;
        if constexpr (LOADS == 2) kbuf[wslot][u1] = DIST == 3 ? pw1 : ld1;

        // epilogue: relu per head; the two heads of a pair are added, then
        // the pair sums in ascending pair order (the head-sum order shared
        // with the small scorer in qsa_small.hip)
        if constexpr (M16) {
            // register u: query quad u/2, column tile u%2; head pair p sits in
            // rows 2*(p%2), 2*(p%2)+1 of row tile (u/2)*NHH + p/2
            #pragma unroll
            for (int p = 0; p < NP; ++p) {
                #pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const floatx4 &c4 = acc16[(u >> 1) * NHH + p / 2][u & 1];
                    const float pp = relu_bits(c4[2 * (p % 2)]) + relu_bits(c4[2 * (p % 2) + 1]);
                    tot[u] = (p == 0) ? pp : tot[u] + pp;
                }
            }
            // v_permlane16_swap of each query quad's two column tiles: lanes
            // 0-31 then hold one query's 32 blocks and lanes 32-63 another's
            // (queries 4*qd + u%2 and 4*qd + u%2 + 2), so every store writes
            // two whole 128-byte row segments, as the 32x32x16 form does
            #pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, tot[2 * qd]),
                                                                 __builtin_bit_cast(uint32_t, tot[2 * qd + 1]), false, false);
                tot[2 * qd] = __builtin_bit_cast(float, static_cast<uint32_t>(sw[0]));
                tot[2 * qd + 1] = __builtin_bit_cast(float, static_cast<uint32_t>(sw[1]));
            }
        } else {
            #pragma unroll
            for (int p = 0; p < NP; ++p) {
                #pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float pp = relu_bits(acc[p][u]) + relu_bits(acc[p][u + 8]);   // heads 2p, 2p+1
                    tot[u] = (!ACCUM && p == 0) ? pp : tot[u] + pp;
                }
            }
        }
        if constexpr (STREAM) {
            stream_tile(tile, tot);
        } else {
            #pragma unroll
            for (int u = 0; u < 8; ++u) {
                if constexpr (BUF) {
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, tot[u]), rs,
                                                          static_cast<int>(rowoff[u] + coloff), 0,
                                                          kStoreNT);
                } else if (rowel[u] >= 0 && coloff != kOut) {
                    __builtin_nontemporal_store(tot[u], srow_base + rowel[u] + bcol);
                }
            }
        }
        __syncthreads();
        slot = nslot;
    };
    for (int tile = tb; tile < te; tile += 2) {
        step(tile, p0, p1, q0, q1);
        if (tile + 1 < te) step(tile + 1, q0, q1, p0, p1);
    }

    if constexpr (TAIL) {
        // The partial block nf, scored by the last split of each query group
        // from the query fragments already in registers, in the fixed order
        // of the tail model: per (query, head) one fp32 fma chain over the
        // channels in ascending order, relu (acc > 0 ? acc : +0), then the
        // heads added in ascending order.  v_permlane32_swap of the fragments
        // of head pairs p0 = 2c and p1 = 2c+1 gives lanes 0-31 whole 16-wide
        // channel runs of pair p0 and lanes 32-63 those of pair p1, so lane l
        // runs the chain of query t_base + l%16, head 4c + l/16 (in the pass).
        if (tail_wg) {   // uniform over the workgroup
          if constexpr (M16) {
            // The same chains from the 16x16x32 fragments.  In K-step s, lane
            // group j (lanes 16j .. 16j+15) of row tile i holds channels
            // 32s + 8j .. +7 of row l%16; a 4x4 transpose over (row tile,
            // lane group) -- v_permlane32_swap between tiles i and i+2, then
            // v_permlane16_swap between i and i+1 -- gives lane group j all
            // 32 channels of its row in tile 4c + j, in channel order.  Lane l
            // so runs the chain of row l%16 of row tile 4c + l/16: query
            // 4*((4c + l/16) / NHH) + (l%16)/4 of the wave, head
            // 4*((4c + l/16) % NHH) + l%4.
            constexpr int NCH = RT / 4;   // chains per lane
            uint4 kc[CHUNKS];
            #pragma unroll
            for (int c = 0; c < CHUNKS; ++c) kc[c] = ktail[c];   // staged at the prologue
            float r[NCH];
            #pragma unroll
            for (int c = 0; c < NCH; ++c) {
                float acc = 0.0f;
                #pragma unroll
                for (int s = 0; s < KS16; ++s) {
                    const uint4 f0 = __builtin_bit_cast(uint4, qa16[4 * c + 0][s]);
                    const uint4 f1 = __builtin_bit_cast(uint4, qa16[4 * c + 1][s]);
                    const uint4 f2 = __builtin_bit_cast(uint4, qa16[4 * c + 2][s]);
                    const uint4 f3 = __builtin_bit_cast(uint4, qa16[4 * c + 3][s]);
                    const uint32_t a0[4] = {f0.x, f0.y, f0.z, f0.w}, a1[4] = {f1.x, f1.y, f1.z, f1.w};
                    const uint32_t a2[4] = {f2.x, f2.y, f2.z, f2.w}, a3[4] = {f3.x, f3.y, f3.z, f3.w};
                    uint32_t ch[4][4];   // [chunk][dword]
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const auto s02 = __builtin_amdgcn_permlane32_swap(a0[e], a2[e], false, false);
                        const auto s13 = __builtin_amdgcn_permlane32_swap(a1[e], a3[e], false, false);
                        const auto lo = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
                        const auto hi = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
                        ch[0][e] = lo[0];
                        ch[1][e] = lo[1];
                        ch[2][e] = hi[0];
                        ch[3][e] = hi[1];
                    }
                    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 k4 = kc[4 * s + j];
                        const uint32_t kw[4] = {k4.x, k4.y, k4.z, k4.w};
                        #pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float q0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ch[j][e] & 0xffffu)));
                            const float q1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(ch[j][e] >> 16)));
                            const float k0f = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kw[e] & 0xffffu)));
                            const float k1f = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kw[e] >> 16)));
                            acc = __builtin_fmaf(k0f, q0, acc);
                            acc = __builtin_fmaf(k1f, q1, acc);
                        }
                    }
                }
                r[c] = acc > 0.0f ? acc : 0.0f;
            }
            // head sum across lanes, through the ring (free after the last
            // barrier): the wave's (query, head) results at 8*query + head
            float *red = reinterpret_cast<float *>(&kbuf[0][0]) + w * (8 * kWaveQueries);
            #pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int i = 4 * c + (l >> 4);
                red[8 * (4 * (i / NHH) + ((l & 15) >> 2)) + 4 * (i % NHH) + (l & 3)] = r[c];
            }
            __syncthreads();
            const int t = t_base + l;
            if (l < kWaveQueries && t < a.nq) {
                float *cell = srow_base + static_cast<int64_t>(t) * a.ld_s + a.nf;
                float sum = 0.0f;
                #pragma unroll
                for (int h = 0; h < 4 * NHH; ++h)
                    if (h < a.nh) sum = sum + red[8 * l + h];
                if (a.tail_add != 0.0f) sum = sum + a.tail_add;   // forced-tail rule
                *cell = sum;
            }
          } else {
            constexpr int NPC = (NP + 1) / 2;
            uint4 kc[CHUNKS];
            #pragma unroll
            for (int c = 0; c < CHUNKS; ++c) kc[c] = ktail[c];   // staged at the prologue
            float r[NPC];
            #pragma unroll
            for (int c = 0; c < NPC; ++c) {
                float acc = 0.0f;
                #pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const uint4 x = __builtin_bit_cast(uint4, qa[2 * c][s]);
                    const uint4 y = 2 * c + 1 < NP ? __builtin_bit_cast(uint4, qa[2 * c + 1 < NP ? 2 * c + 1 : 0][s])
                                                   : make_uint4(0, 0, 0, 0);
                    const auto sw0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
                    const auto sw1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
                    const auto sw2 = __builtin_amdgcn_permlane32_swap(x.z, y.z, false, false);
                    const auto sw3 = __builtin_amdgcn_permlane32_swap(x.w, y.w, false, false);
                    // channels 16s .. 16s+7, then 16s+8 .. 16s+15
                    const uint32_t qw[8] = {sw0[0], sw1[0], sw2[0], sw3[0], sw0[1], sw1[1], sw2[1], sw3[1]};
                    const uint4 k0 = kc[2 * s], k1 = kc[2 * s + 1];
                    const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                    #pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float q0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(qw[e] & 0xffffu)));
                        const float q1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(qw[e] >> 16)));
                        const float k0f = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kw[e] & 0xffffu)));
                        const float k1f = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(kw[e] >> 16)));
                        acc = __builtin_fmaf(k0f, q0, acc);
                        acc = __builtin_fmaf(k1f, q1, acc);
                    }
                }
                r[c] = acc > 0.0f ? acc : 0.0f;
            }
            // head sum across lanes: the ring is free after the last barrier
            float *red = reinterpret_cast<float *>(&kbuf[0][0]) + w * (NPC * 64);
            #pragma unroll
            for (int c = 0; c < NPC; ++c) red[64 * c + l] = r[c];
            __syncthreads();
            const int t = t_base + l;
            if constexpr (STREAM) {
                // lane r < 16: row r's tail score, a candidate like any other
                // (the block of the largest id, so it goes last)
                float sum = 0.0f;
                #pragma unroll
                for (int c = 0; c < NPC; ++c) {
                    #pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (4 * c + j < a.nh) sum = sum + red[64 * c + 16 * j + (l & 15)];
                }
                if (a.tail_add != 0.0f) sum = sum + a.tail_add;   // forced-tail rule
                stream_tail(sum);
            } else if (l < kWaveQueries && t < a.nq) {
                float *cell = srow_base + static_cast<int64_t>(t) * a.ld_s + a.nf;
                float sum = ACCUM ? *cell : 0.0f;
                #pragma unroll
                for (int c = 0; c < NPC; ++c) {
                    #pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (4 * c + j < a.nh) sum = sum + red[64 * c + 16 * j + l];
                }
                if (a.tail_add != 0.0f) sum = sum + a.tail_add;   // forced-tail rule
                *cell = sum;
            }
          }
        }
    }

    if constexpr (STREAM) {
        // Each row's selection from its buffer, the wave's rows one after
        // another (the ring is free: every wave has passed its last barrier).
        uint64_t *slot = reinterpret_cast<uint64_t *>(&kbuf[1][0]) + wu * 128;
        const int nrows = min(kWaveQueries, a.nq - t_base);   // uniform
        uint32_t cv = 0;
        #pragma unroll
        for (int r = 0; r < kWaveQueries; ++r) cv = lane_set(cv, l, r, cnt[r]);
        for (int r = 0; r < nrows; ++r) {
            const int64_t drow = static_cast<int64_t>(g) * a.dst_group_rows + a.dst_row0 + t_base + r;
            stream_final(wval + r * kStreamCap, wid + r * kStreamCap,
                         __builtin_amdgcn_readlane(cv, r), a.k, kk, wkb[r], slot, a.ids + drow * a.ld_ids,
                         a.vals ? a.vals + drow * a.ld_ids : nullptr, l);
        }
    }

    if constexpr (SEL > 0) {
        // The wave's score stores (its 16 rows, every block) before its own
        // loads of them: the stores were made by other lanes of this wave.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const int nrows = min(kWaveQueries, a.nq - t_base);   // uniform
        auto row = [&](int i) { return srow_base + static_cast<int64_t>(t_base + i) * a.ld_s; };
        auto select = [&](int i, const uint32_t (&x)[SEL]) __attribute__((always_inline)) {
            const int64_t drow = static_cast<int64_t>(g) * a.dst_group_rows + a.dst_row0 + t_base + i;
            topk_row_select<SEL, true>(row(i), a.nb, a.k, x, a.ids + drow * a.ld_ids,
                                       a.vals ? a.vals + drow * a.ld_ids : nullptr, sel_slot[wu],
                                       sel_stash[wu], l);
        };
        // two register sets: the next row's loads are in flight while the
        // current row is selected
        uint32_t xa[SEL], xb[SEL];
        if (nrows > 0) topk_row_load<SEL>(row(0), a.nb, l, xa);
        for (int i = 0; i < nrows; i += 2) {
            if (i + 1 < nrows) topk_row_load<SEL>(row(i + 1), a.nb, l, xb);
            select(i, xa);
            if (i + 1 >= nrows) break;
            if (i + 2 < nrows) topk_row_load<SEL>(row(i + 2), a.nb, l, xa);
            select(i + 1, xb);
        }
    }
}

typedef void (*score_fn)(ScoreArgs);

// Heads per pass: 8 keep the resident queries (128 VGPRs at D = 128), four
// accumulators and the staging registers inside 256 VGPRs, i.e. two waves
// per SIMD; more heads take a second, accumulating pass.
constexpr int kHeadsPerPass = 8;

// One head pass with buffer stores takes the 16x16x32 form (M16 = BUF).
template <int D, bool BUF, bool TAIL, bool SRC32>
score_fn pick_d(int np, bool accum) {
    switch (np) {
        case 1: return accum ? score_full_kernel<D, 1, true, BUF, TAIL, SRC32> : score_full_kernel<D, 1, false, BUF, TAIL, SRC32, 0, false, BUF>;
        case 2: return accum ? score_full_kernel<D, 2, true, BUF, TAIL, SRC32> : score_full_kernel<D, 2, false, BUF, TAIL, SRC32, 0, false, BUF>;
        case 3: return accum ? score_full_kernel<D, 3, true, BUF, TAIL, SRC32> : score_full_kernel<D, 3, false, BUF, TAIL, SRC32, 0, false, BUF>;
        case 4: return accum ? score_full_kernel<D, 4, true, BUF, TAIL, SRC32> : score_full_kernel<D, 4, false, BUF, TAIL, SRC32, 0, false, BUF>;
    }
    return nullptr;
}

template <int D, bool SRC32>
score_fn pick_dt(int np, bool accum, bool buf, bool tail) {
    if (tail) return buf ? pick_d<D, true, true, SRC32>(np, accum) : pick_d<D, false, true, SRC32>(np, accum);
    return buf ? pick_d<D, true, false, SRC32>(np, accum) : pick_d<D, false, false, SRC32>(np, accum);
}

score_fn pick(int D, int np, bool accum, bool buf, bool tail, bool src32) {
    if (D == 128) return src32 ? pick_dt<128, true>(np, accum, buf, tail) : pick_dt<128, false>(np, accum, buf, tail);
    if (D == 64) return src32 ? pick_dt<64, true>(np, accum, buf, tail) : pick_dt<64, false>(np, accum, buf, tail);
    return nullptr;
}

// The fused-selection instances: one head pass (np <= 4), buffer stores, and
// rows whose 64-wide column count takes the selector's 16- or 33-column case
// (9-16 columns: 513-1024 blocks; 33 columns: 2049-2112 blocks).
template <int D, bool TAIL, bool SRC32, int SEL>
score_fn pick_sel_np(int np) {
    switch (np) {
        case 1: return score_full_kernel<D, 1, false, true, TAIL, SRC32, SEL>;
        case 2: return score_full_kernel<D, 2, false, true, TAIL, SRC32, SEL>;
        case 3: return score_full_kernel<D, 3, false, true, TAIL, SRC32, SEL>;
        case 4: return score_full_kernel<D, 4, false, true, TAIL, SRC32, SEL>;
    }
    return nullptr;
}

template <int D, int SEL>
score_fn pick_sel_ts(int np, bool tail, bool src32) {
    if (tail) return src32 ? pick_sel_np<D, true, true, SEL>(np) : pick_sel_np<D, true, false, SEL>(np);
    return src32 ? pick_sel_np<D, false, true, SEL>(np) : pick_sel_np<D, false, false, SEL>(np);
}

// The streaming-selection instances: one head pass (np <= 4).
template <int D, bool TAIL, bool SRC32>
score_fn pick_stream_np(int np) {
    switch (np) {
        case 1: return score_full_kernel<D, 1, false, true, TAIL, SRC32, 0, true>;
        case 2: return score_full_kernel<D, 2, false, true, TAIL, SRC32, 0, true>;
        case 3: return score_full_kernel<D, 3, false, true, TAIL, SRC32, 0, true>;
        case 4: return score_full_kernel<D, 4, false, true, TAIL, SRC32, 0, true>;
    }
    return nullptr;
}

template <int D>
score_fn pick_stream_ts(int np, bool tail, bool src32) {
    if (tail) return src32 ? pick_stream_np<D, true, true>(np) : pick_stream_np<D, true, false>(np);
    return src32 ? pick_stream_np<D, false, true>(np) : pick_stream_np<D, false, false>(np);
}

score_fn pick_stream(int D, int np, bool tail, bool src32) {
    if (D == 128) return pick_stream_ts<128>(np, tail, src32);
    if (D == 64) return pick_stream_ts<64>(np, tail, src32);
    return nullptr;
}

// Columns of the fused selection for nb blocks (0: no fused form).
int sel_columns(int64_t nb) {
    const int64_t nj = (nb + 63) / 64;
    if (nj > 8 && nj <= 16) return 16;
    if (nj == 33) return 33;
    return 0;
}

score_fn pick_sel(int D, int np, bool tail, bool src32, int sel) {
    if (D == 128) return sel == 16 ? pick_sel_ts<128, 16>(np, tail, src32) : pick_sel_ts<128, 33>(np, tail, src32);
    if (D == 64) return sel == 16 ? pick_sel_ts<64, 16>(np, tail, src32) : pick_sel_ts<64, 33>(np, tail, src32);
    return nullptr;
}

// Splits of the block axis so that base * splits workgroups reach target
// (at most one split per tile); returns the splits and the tiles per split.
void split_blocks(int64_t base, int64_t n_tiles, int64_t target, int64_t *splits, int64_t *tps) {
    int64_t sp = 1;
    if (base < target) {
        sp = (target + base - 1) / base;
        if (sp > n_tiles) sp = n_tiles;
        if (sp < 1) sp = 1;
    }
    *tps = (n_tiles + sp - 1) / sp;
    *splits = (n_tiles + *tps - 1) / *tps;
}

// The wide scorer's grid: groups of 64 queries per workgroup over the KV
// heads, the block axis split only when the groups cannot fill the CUs twice
// (512 workgroups).
struct WideGrid {
    int64_t n_tiles, n_qgroups, base, splits, tps;
};

WideGrid wide_grid(const ScoreGeom &geo) {
    WideGrid w;
    w.n_tiles = (geo.nf + kTileBlocks - 1) / kTileBlocks;
    w.n_qgroups = (geo.nq + kGroupQueries - 1) / kGroupQueries;
    w.base = static_cast<int64_t>(geo.G) * w.n_qgroups;
    w.splits = 1;
    w.tps = w.n_tiles;
    split_blocks(w.base, w.n_tiles, 512, &w.splits, &w.tps);
    return w;
}

}  // namespace

bool stream_select_serves(const ScoreGeom &geo, bool tail) {
    if (geo.nf <= 0 || geo.nq <= 0 || geo.G <= 0 || geo.H > kHeadsPerPass) return false;
    if (decode_rows(geo) || small_rows(geo)) return false;
    // block ids are kept as 16 bits
    if (geo.nf + (tail ? 1 : 0) > 65536) return false;
    // one workgroup per query group over all blocks
    const WideGrid w = wide_grid(geo);
    return w.splits == 1 && w.base <= 0x7fffffffLL;
}

hipError_t launch_score_full(const ScoreGeom &geo, bool tail, hipStream_t s, const float *q32,
                             uint16_t *q16w, const FusedSelect *fs, bool *selected) {
    if (selected) *selected = false;
    if (geo.nf <= 0 || geo.nq <= 0 || geo.G <= 0) return hipSuccess;
    if (small_rows(geo)) return launch_score_small(geo, tail, s, q32, q16w);
    const int hpp = kHeadsPerPass;
    // buffer stores address one KV head's rows with 32-bit offsets below 2^30
    const bool buf = static_cast<int64_t>(geo.nq) * geo.ld_s * 4 < (int64_t(1) << 30);
    const WideGrid wg = wide_grid(geo);
    const int64_t n_tiles = wg.n_tiles, n_qgroups = wg.n_qgroups, splits = wg.splits, tps = wg.tps;
    if (n_tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int64_t grid = wg.base * splits;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;

    // fused selection: each workgroup scores every block of its query group
    const int64_t nb = geo.nf + (tail ? 1 : 0);
    // streaming selection: no score is written
    if (fs && fs->stream && fs->k > 0 && stream_select_serves(geo, tail)) {
        const int np = (geo.H + 1) / 2;
        score_fn fn = pick_stream(geo.D, np, tail, q32 != nullptr);
        if (!fn) return hipErrorInvalidValue;
        ScoreArgs a{geo.q16, q32, q32 ? q16w : nullptr, geo.qts, geo.kblk, geo.khs, nullptr,
                    geo.ld_s, geo.G, geo.nq, geo.H, 0, geo.H, 0, geo.nf,
                    static_cast<int32_t>(n_qgroups), 1, static_cast<int32_t>(tps),
                    static_cast<int32_t>(n_tiles), geo.tail_add, fs->ids, fs->ld_ids, fs->vals,
                    fs->k, static_cast<int32_t>(nb), fs->dst_group_rows, fs->dst_row0};
        void *args[] = {&a};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn),
                                       dim3(static_cast<unsigned>(grid)), dim3(256), args, 0, s);
        if (e == hipSuccess && selected) *selected = true;
        return e;
    }
    const int sel = fs && fs->fused && fs->k > 0 ? sel_columns(nb) : 0;
    if (sel > 0 && splits == 1 && geo.H <= hpp && buf) {
        const int np = (geo.H + 1) / 2;
        score_fn fn = pick_sel(geo.D, np, tail, q32 != nullptr, sel);
        if (!fn) return hipErrorInvalidValue;
        ScoreArgs a{geo.q16, q32, q32 ? q16w : nullptr, geo.qts, geo.kblk, geo.khs, geo.scores,
                    geo.ld_s, geo.G, geo.nq, geo.H, 0, geo.H, 0, geo.nf,
                    static_cast<int32_t>(n_qgroups), 1, static_cast<int32_t>(tps),
                    static_cast<int32_t>(n_tiles), geo.tail_add, fs->ids, fs->ld_ids, fs->vals,
                    fs->k, static_cast<int32_t>(nb), fs->dst_group_rows, fs->dst_row0};
        void *args[] = {&a};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn),
                                       dim3(static_cast<unsigned>(grid)), dim3(256), args, 0, s);
        if (e == hipSuccess && selected) *selected = true;
        return e;
    }

    for (int h0 = 0; h0 < geo.H; h0 += hpp) {
        const int nh = (geo.H - h0 < hpp) ? geo.H - h0 : hpp;
        const int np = (nh + 1) / 2;
        score_fn fn = pick(geo.D, np, h0 > 0, buf, tail, q32 != nullptr);
        if (!fn) return hipErrorInvalidValue;
        ScoreArgs a{geo.q16, q32, q32 ? q16w : nullptr, geo.qts, geo.kblk, geo.khs, geo.scores, geo.ld_s,
                    geo.G, geo.nq, geo.H, h0, nh, h0 > 0 ? 1 : 0, geo.nf,
                    static_cast<int32_t>(n_qgroups), static_cast<int32_t>(splits),
                    static_cast<int32_t>(tps), static_cast<int32_t>(n_tiles),
                    h0 + nh == geo.H ? geo.tail_add : 0.0f, nullptr, 0, nullptr, 0, 0, 0, 0};
        void *args[] = {&a};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn),
                                       dim3(static_cast<unsigned>(grid)), dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qsa
