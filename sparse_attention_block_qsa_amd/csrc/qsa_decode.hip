// qsa_decode.hip -- the QSA block scorer for decode steps: at most one MFMA
// row block of queries per KV head (QPG = 16/NP queries: 4 at H = 8, 8 at
// H <= 4, 2 at H > 8), e.g. one new query per KV head per step.
//
// score(g, t, b) = sum_h relu( sum_i k[g, b, i] * q[t, g, h, i] )
// (Strata pull request #228, part 1, score formula.)
//
// The small scorer (qsa_small.hip) stages each 32-block K tile through LDS
// for the four query groups of a workgroup; with one query group per KV head
// three of its four waves hold no query and every tile costs an LDS round
// trip and a barrier.  Here one wave scores one 32-block tile of one KV head,
// one wave per workgroup:
//  * the B operand is read straight from memory into the fragment layout
//    (lane l holds k[b0 + l%32][16s + 8*(l/32) .. +7] for K-step s: 16-byte
//    loads, each 32-lane half reading 32 block rows), no LDS and no barrier;
//  * the A operand is the small scorer's: the QPG queries x 2*NP heads of
//    the KV head in one 32-row block, loaded per lane (fp32 queries converted
//    on load with the conversion kernel's instruction; the wave of tile 0
//    writes the fp16 bits to the caller's buffer when there is one);
//  * the MFMA sequence (v_mfma_f32_32x32x16_f16, K-steps ascending) and the
//    epilogue (relu per head, v_permlane32_swap pairing, pair sums in
//    ascending pair order) are the small scorer's, so the bits are the same;
//  * every load of a wave is issued before its first MFMA: a tile costs one
//    memory latency;
//  * the partial last block, when there is one, is scored by one more wave
//    per KV head in the fixed order of the tail model (one lane per (query,
//    head) chain, the heads then added in ascending order through LDS).
// HBM-bound: 2*D bytes of keys per block, read once; the queries (H*D per
// query row) are read by every wave of their KV head, from L2.
#include "qsa_internal.h"

#pragma clang fp contract(off)

namespace qsa {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct DecodeArgs {
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
    int32_t n_tiles;       // 32-block tiles over the full blocks
    int32_t tail;          // block nf is a partial block: one more wave per KV head
    float tail_add;        // added to the partial block's score when nonzero
};

__device__ __forceinline__ float relu_bits(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int32_t, x), 0));
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

template <int D, int NP, bool SRC32>
__global__ __launch_bounds__(64) void score_decode_kernel(DecodeArgs a) {
    constexpr int KS = D / 16;
    constexpr int QPG = 16 / NP;
    static_assert(NP == 1 || NP == 2 || NP == 4 || NP == 8, "head pairs per row block");
    __shared__ float red[QPG][2 * NP];

    const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
    const int per_g = a.n_tiles + a.tail;
    const int g = static_cast<int>(L / per_g);
    const int item = static_cast<int>(L % per_g);
    const bool tail_item = item == a.n_tiles;   // uniform
    const int l = threadIdx.x;

    // ---- A operand: this lane's (query, head) row, channels 16s + 8*(l/32) ..
    const int R = l & 31, kc = l >> 5;
    const int c = 4 * (R >> 3) + (R & 3);
    const int p_in = c / QPG, q_in = c % QPG;
    const int h_in = 2 * p_in + ((R >> 2) & 1);
    const bool a_ok = q_in < a.nq && h_in < a.H;
    const int64_t a_off = static_cast<int64_t>(a_ok ? q_in : 0) * a.qts +
                          static_cast<int64_t>(g * a.H + (a_ok ? h_in : 0)) * D + 8 * kc;
    const uint16_t *kg = a.kblk + static_cast<int64_t>(g) * a.khs;

    // ---- the keys first: the tile's B fragments, or the partial block's key
    // (blocks past nf repeat block nf-1: their output columns are not stored)
    uint4 kv[KS][2];
    if (!tail_item) {
        const int64_t b = min(static_cast<int64_t>(item) * kTileBlocks + (l & 31), a.nf - 1);
        #pragma unroll
        for (int s = 0; s < KS; ++s)
            kv[s][0] = *reinterpret_cast<const uint4 *>(kg + b * D + 16 * s + 8 * kc);
    } else {
        const uint16_t *kt = kg + a.nf * D;
        #pragma unroll
        for (int s = 0; s < KS; ++s) {
            kv[s][0] = *reinterpret_cast<const uint4 *>(kt + 16 * s);
            kv[s][1] = *reinterpret_cast<const uint4 *>(kt + 16 * s + 8);
        }
    }

    // ---- the queries
    half8 qa[KS];
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
        if (a.q16w && item == 0 && a_ok) {
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
    float *sbase = a.scores + static_cast<int64_t>(g) * a.nq * a.ld_s;

    if (!tail_item) {
        floatx16 acc = {};
        #pragma unroll
        for (int s = 0; s < KS; ++s)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[s], __builtin_bit_cast(half8, kv[s][0]),
                                                         s == 0 ? floatx16{} : acc, 0, 0, 0);
        // relu per head, then the two heads of each pair into one lane (the
        // swap gives lanes 0-31 both heads of query q and lanes 32-63 those
        // of q+1); pair sums in ascending pair order
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
                    __builtin_bit_cast(uint32_t, pr[r]), __builtin_bit_cast(uint32_t, pr[r + 1]),
                    false, false);
                const float pair = __builtin_bit_cast(float, static_cast<uint32_t>(sw[0])) +
                                   __builtin_bit_cast(float, static_cast<uint32_t>(sw[1]));
                tot[m] = p == 0 ? pair : tot[m] + pair;
            }
        }
        const int64_t b = static_cast<int64_t>(item) * kTileBlocks + (l & 31);
        #pragma unroll
        for (int m = 0; m < QPG / 2; ++m) {
            const int t = 2 * m + kc;
            if (t < a.nq && b < a.nf) sbase[static_cast<int64_t>(t) * a.ld_s + b] = tot[m];
        }
    } else {
        // the partial block nf: lane l < 32 runs the chain of its A row R = l;
        // v_permlane32_swap gives it the other half of every 16-channel run
        // (held by lane l + 32), so it walks channels ascending
        float acc = 0.0f;
        #pragma unroll
        for (int s = 0; s < KS; ++s) {
            const uint4 x = __builtin_bit_cast(uint4, qa[s]);
            const auto w0 = __builtin_amdgcn_permlane32_swap(x.x, x.x, false, false);
            const auto w1 = __builtin_amdgcn_permlane32_swap(x.y, x.y, false, false);
            const auto w2 = __builtin_amdgcn_permlane32_swap(x.z, x.z, false, false);
            const auto w3 = __builtin_amdgcn_permlane32_swap(x.w, x.w, false, false);
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
        if (l < 32) red[q_in][h_in] = r;   // padded heads and rows hold +0
        __syncthreads();
        if (l < QPG && l < a.nq) {
            float sum = 0.0f;
            for (int h = 0; h < a.H; ++h) sum = sum + red[l][h];
            if (a.tail_add != 0.0f) sum = sum + a.tail_add;   // forced-tail rule
            sbase[static_cast<int64_t>(l) * a.ld_s + a.nf] = sum;
        }
    }
}

typedef void (*decode_fn)(DecodeArgs);

template <int D, bool SRC32>
decode_fn pick_np(int np) {
    switch (np) {
        case 1: return score_decode_kernel<D, 1, SRC32>;
        case 2: return score_decode_kernel<D, 2, SRC32>;
        case 4: return score_decode_kernel<D, 4, SRC32>;
        case 8: return score_decode_kernel<D, 8, SRC32>;
    }
    return nullptr;
}

// Head pairs per MFMA row block: the smallest of 1, 2, 4, 8 that holds H
// (the small scorer's choice, so that both produce the same bits).
int decode_pairs(int H) {
    const int np = (H + 1) / 2;
    return np <= 1 ? 1 : np <= 2 ? 2 : np <= 4 ? 4 : 8;
}

}  // namespace

bool decode_rows(const ScoreGeom &g) {
    return g.nq > 0 && g.nq <= 16 / decode_pairs(g.H) && g.nf > 0;
}

hipError_t launch_score_decode(const ScoreGeom &geo, bool tail, hipStream_t s, const float *q32,
                               uint16_t *q16w) {
    if (!decode_rows(geo) || geo.G <= 0) return hipErrorInvalidValue;
    const int np = decode_pairs(geo.H);
    const int64_t n_tiles = (geo.nf + kTileBlocks - 1) / kTileBlocks;
    const int64_t grid = static_cast<int64_t>(geo.G) * (n_tiles + (tail ? 1 : 0));
    if (grid > 0x7fffffffLL || n_tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    decode_fn fn = nullptr;
    if (geo.D == 128) fn = q32 ? pick_np<128, true>(np) : pick_np<128, false>(np);
    else if (geo.D == 64) fn = q32 ? pick_np<64, true>(np) : pick_np<64, false>(np);
    if (!fn) return hipErrorInvalidValue;
    DecodeArgs a{geo.q16, q32, q32 ? q16w : nullptr, geo.qts, geo.kblk, geo.khs, geo.scores,
                 geo.ld_s, geo.G, geo.nq, geo.H, geo.nf, static_cast<int32_t>(n_tiles),
                 tail ? 1 : 0, geo.tail_add};
    void *args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(static_cast<unsigned>(grid)),
                           dim3(64), args, 0, s);
}

}  // namespace qsa
