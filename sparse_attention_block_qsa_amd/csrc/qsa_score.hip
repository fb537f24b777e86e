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
//    staged once per workgroup in LDS, double-buffered, stored in fragment
//    order so that every ds_read_b128 is lane-contiguous, and reused by the
//    four waves and by every head pair.
//  * The 32x32 accumulator of one head pair holds, per lane, the same
//    (query, block) cells for both heads (registers r and r+8), so the relu
//    and the head sum are lane-local: tot[u] += relu(acc[u]); tot[u] +=
//    relu(acc[u+8]), heads ascending.  Two waves per SIMD (<= 256 VGPRs each)
//    let one wave's relu/add epilogue run on the VALU while the matrix core
//    works on the other wave's MFMAs.
//  * Stores: for a fixed accumulator register the 64 lanes hold 2 query rows
//    x 32 consecutive blocks, i.e. two full 128-byte row segments.
//  * Ragged edges: query rows >= nq load zeros, blocks >= nf repeat block
//    nf-1 (MFMA output columns are independent, and those columns are never
//    stored), and stores are masked, so the write set is exactly
//    scores[g*nq + t][0, nf).
//  * Grid: (KV head, 64-query group, block split), with logical ids laid out
//    so that each XCD (blockIdx % 8) takes a contiguous range: the splits of
//    one query group and the query groups of one KV head share that XCD's L2.
#include "qsa_internal.h"

namespace qsa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct ScoreArgs {
    const uint16_t *q16;
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
};

// Logical workgroup id such that the workgroups the hardware places on one
// XCD (consecutive ids modulo 8 land on consecutive XCDs) get a contiguous
// logical range.  Bijective for any grid size.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t bid, uint32_t nblk) {
    const uint32_t q = nblk / 8, r = nblk % 8;
    const uint32_t x = bid % 8, idx = bid / 8;
    return x * q + (x < r ? x : r) + idx;
}

// relu on fp32 bits: as signed integers, negative floats (and -0) are < 0 and
// non-negative floats keep their order, so max(bits, 0) is relu(x) with -0
// mapped to +0.  One v_max_i32, no NaN canonicalisation.
__device__ __forceinline__ float relu_bits(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int32_t, x), 0));
}

template <int D, int NP, bool ACCUM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void score_full_kernel(ScoreArgs a) {
    constexpr int KS = D / 16;              // MFMA K-steps per head
    constexpr int CHUNKS = D / 8;           // 16-byte chunks per block row
    constexpr int TILE_U4 = CHUNKS * kTileBlocks;
    constexpr int LOADS = TILE_U4 / 256;    // uint4 per thread per tile
    constexpr int PB = NP < 4 ? NP : 4;     // accumulators live at once (16 VGPRs each)
    static_assert(TILE_U4 % 256 == 0, "tile must split evenly over 256 threads");

    __shared__ uint4 kbuf[2][TILE_U4];

    const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    const int split = static_cast<int>(L % a.n_splits);
    const uint32_t rest = L / a.n_splits;
    const int qg = static_cast<int>(rest % a.n_qgroups);
    const int g = static_cast<int>(rest / a.n_qgroups);

    const int tile_begin = split * a.tiles_per_split;
    const int tile_end = min(a.n_tiles, tile_begin + a.tiles_per_split);
    if (tile_begin >= tile_end) return;   // uniform over the workgroup

    const int w = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int t_base = qg * kGroupQueries + w * kWaveQueries;

    // ---- stationary query fragments --------------------------------------
    half8 qa[NP][KS];
    {
        const int tq = l & 15, hh = (l >> 4) & 1, kc = l >> 5;
        const int t = t_base + tq;
        #pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int h = 2 * p + hh;
            const bool valid = (t < a.nq) && (h < a.nh);
            const uint16_t *src = a.q16 + static_cast<int64_t>(valid ? t : 0) * a.qts +
                                  static_cast<int64_t>(g * a.H + a.h0 + (valid ? h : 0)) * D +
                                  8 * kc;
            #pragma unroll
            for (int s = 0; s < KS; ++s) {
                half8 v = {};
                if (valid) v = *reinterpret_cast<const half8 *>(src + 16 * s);
                qa[p][s] = v;
            }
        }
    }

    // ---- cooperative K tile staging --------------------------------------
    // Each thread moves LOADS (1 or 2) 16-byte chunks per tile; LDS index
    // u = threadIdx.x + 256*c is chunk-major (u = chunk*32 + block), which is
    // also the MFMA B-fragment order: lane l of K-step s reads u = 64*s + l.
    // Plain scalars (no array, no lambda) keep the staging in VGPRs.
    static_assert(LOADS == 1 || LOADS == 2, "D must be 64 or 128");
    const uint16_t *kg = a.kblk + static_cast<int64_t>(g) * a.khs;
    const int u0 = threadIdx.x, u1 = threadIdx.x + 256;
    const int off0 = 8 * (u0 / kTileBlocks), off1 = 8 * (u1 / kTileBlocks);
    const int bb0 = u0 % kTileBlocks, bb1 = u1 % kTileBlocks;
    const int64_t last = a.nf - 1;
    // Blocks past nf only feed MFMA output columns that are never stored, so
    // their rows may be any in-bounds data: clamp to the last full block.
    uint4 kr0, kr1 = make_uint4(0, 0, 0, 0);
    {
        const int64_t b0 = static_cast<int64_t>(tile_begin) * kTileBlocks;
        kr0 = *reinterpret_cast<const uint4 *>(kg + min(b0 + bb0, last) * D + off0);
        if constexpr (LOADS == 2)
            kr1 = *reinterpret_cast<const uint4 *>(kg + min(b0 + bb1, last) * D + off1);
        kbuf[0][u0] = kr0;
        if constexpr (LOADS == 2) kbuf[0][u1] = kr1;
    }
    __syncthreads();

    float *srow_base = a.scores + static_cast<int64_t>(g) * a.nq * a.ld_s;
    const int bl = l & 31;

    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int cur = (tile - tile_begin) & 1;
        const bool more = tile + 1 < tile_end;
        if (more) {
            const int64_t b0 = static_cast<int64_t>(tile + 1) * kTileBlocks;
            kr0 = *reinterpret_cast<const uint4 *>(kg + min(b0 + bb0, last) * D + off0);
            if constexpr (LOADS == 2)
                kr1 = *reinterpret_cast<const uint4 *>(kg + min(b0 + bb1, last) * D + off1);
        }

        const int64_t bcol = static_cast<int64_t>(tile) * kTileBlocks + bl;
        const bool col_ok = bcol < a.nf;

        float tot[8];
        #pragma unroll
        for (int u = 0; u < 8; ++u) {
            tot[u] = 0.0f;
            if constexpr (ACCUM) {
                const int t = t_base + 8 * (u >> 2) + 4 * (l >> 5) + (u & 3);
                if (t < a.nq && col_ok) tot[u] = srow_base[static_cast<int64_t>(t) * a.ld_s + bcol];
            }
        }

        // Head pairs in batches of PB accumulators; inside a batch the K-step
        // is the outer loop, so the PB MFMAs that consume one B fragment are
        // independent of each other, and the next fragment's LDS read is in
        // flight while they run.
        const uint4 *kcur = &kbuf[cur][l];
        #pragma unroll
        for (int p0 = 0; p0 < NP; p0 += PB) {
            floatx16 acc[PB];
            half8 kf = __builtin_bit_cast(half8, kcur[0]);
            #pragma unroll
            for (int s = 0; s < KS; ++s) {
                half8 kn = kf;
                if (s + 1 < KS) kn = __builtin_bit_cast(half8, kcur[64 * (s + 1)]);
                #pragma unroll
                for (int j = 0; j < PB; ++j) {
                    if (p0 + j < NP) {
                        const floatx16 c = (s == 0) ? floatx16{} : acc[j];
                        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[p0 + j][s], kf, c, 0, 0, 0);
                    }
                }
                kf = kn;
            }
            #pragma unroll
            for (int j = 0; j < PB; ++j) {
                if (p0 + j < NP) {
                    #pragma unroll
                    for (int u = 0; u < 8; ++u) tot[u] += relu_bits(acc[j][u]);       // head 2p
                    #pragma unroll
                    for (int u = 0; u < 8; ++u) tot[u] += relu_bits(acc[j][u + 8]);   // head 2p+1
                }
            }
        }

        // Publish the prefetched tile before issuing this tile's stores: the
        // wait for its loads then does not also wait for the stores.
        if (more) {
            kbuf[cur ^ 1][u0] = kr0;
            if constexpr (LOADS == 2) kbuf[cur ^ 1][u1] = kr1;
        }

        #pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int t = t_base + 8 * (u >> 2) + 4 * (l >> 5) + (u & 3);
            if (t < a.nq && col_ok) srow_base[static_cast<int64_t>(t) * a.ld_s + bcol] = tot[u];
        }
        __syncthreads();
    }
}

typedef void (*score_fn)(ScoreArgs);

// Heads per pass: 12 at D = 64 and 8 at D = 128 keep the resident queries,
// four accumulators and the staging registers inside 256 VGPRs (two waves per
// SIMD); more heads take a second, accumulating pass.
constexpr int heads_per_pass(int D) { return D == 64 ? 12 : 8; }

score_fn pick(int D, int np, bool accum) {
#define QSA_SCORE_CASE(DD, N) \
    if (D == DD && np == N) return accum ? score_full_kernel<DD, N, true> : score_full_kernel<DD, N, false>;
    QSA_SCORE_CASE(128, 1)
    QSA_SCORE_CASE(128, 2)
    QSA_SCORE_CASE(128, 3)
    QSA_SCORE_CASE(128, 4)
    QSA_SCORE_CASE(64, 1)
    QSA_SCORE_CASE(64, 2)
    QSA_SCORE_CASE(64, 3)
    QSA_SCORE_CASE(64, 4)
    QSA_SCORE_CASE(64, 5)
    QSA_SCORE_CASE(64, 6)
#undef QSA_SCORE_CASE
    return nullptr;
}

}  // namespace

hipError_t launch_score_full(const ScoreGeom &geo, hipStream_t s) {
    if (geo.nf <= 0 || geo.nq <= 0 || geo.G <= 0) return hipSuccess;
    const int hpp = heads_per_pass(geo.D);
    const int64_t n_tiles = (geo.nf + kTileBlocks - 1) / kTileBlocks;
    const int64_t n_qgroups = (geo.nq + kGroupQueries - 1) / kGroupQueries;
    const int64_t base = static_cast<int64_t>(geo.G) * n_qgroups;
    // Splits along the block axis only when the query groups alone cannot
    // fill the 256 CUs (two resident workgroups each); keep >= 2 tiles per
    // split so the K-tile pipeline has something to overlap.
    int64_t splits = 1;
    if (base < 512) {
        splits = (512 + base - 1) / base;
        const int64_t max_splits = (n_tiles + 1) / 2;
        if (splits > max_splits) splits = max_splits;
        if (splits < 1) splits = 1;
    }
    const int64_t tps = (n_tiles + splits - 1) / splits;
    splits = (n_tiles + tps - 1) / tps;
    const int64_t grid = base * splits;
    if (grid > 0x7fffffffLL || n_tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;

    for (int h0 = 0; h0 < geo.H; h0 += hpp) {
        const int nh = (geo.H - h0 < hpp) ? geo.H - h0 : hpp;
        const int np = (nh + 1) / 2;
        score_fn fn = pick(geo.D, np, h0 > 0);
        if (!fn) return hipErrorInvalidValue;
        ScoreArgs a{geo.q16, geo.qts, geo.kblk, geo.khs, geo.scores, geo.ld_s,
                    geo.G, geo.nq, geo.H, h0, nh, h0 > 0 ? 1 : 0, geo.nf,
                    static_cast<int32_t>(n_qgroups), static_cast<int32_t>(splits),
                    static_cast<int32_t>(tps), static_cast<int32_t>(n_tiles)};
        void *args[] = {&a};
        hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn),
                                       dim3(static_cast<unsigned>(grid)), dim3(256), args, 0, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace qsa
