// qsa_attention.hip -- attention over the selected blocks: the step after
// the select phase.
//
// The pages stop at the selection (Strata pull request #228, part 1: the
// phase keeps, per query, the blocks whose score ranks in the top k).  The
// reading taken for the step that consumes it is plain softmax attention of
// every query head over the tokens of the blocks its (KV head, query) row
// selected:
//   s_j = scale * sum_i q[t][g][h][i] * k[j][g][i],   scale = fp32(1/sqrt(D))
//   out[t][g][h][:] = sum_j exp(s_j - max) v[j][g][:] / sum_j exp(s_j - max)
// with fp16 queries, keys and values and fp32 arithmetic.
//
// Mapping: one workgroup of 8 waves per (KV head, query) row.  The row's
// selected blocks are cut into chunks of at most 64 tokens; wave w takes
// chunks w, w + 8, ...  Per chunk:
//   * the logits of every head are two MFMA chains (v_mfma_f32_32x32x16_f16,
//     A = 32 tokens' keys loaded straight into fragment layout, B = the
//     row's queries, transposed, from LDS): fp16 products are exact and the
//     sums fp32; lane l receives head l%32's logits of 32 tokens;
//   * head h's chunk maximum and weight sum take the lane's 32 tokens and
//     its partner's (lane l ^ 32); the running maximum, denominator and
//     output are rescaled when the maximum grows (online softmax); the
//     weights go to LDS;
//   * the weighted sum, up to 8 heads, on the matrix cores
//     (v_mfma_f32_16x16x32_f16): each weight scaled by 2^14 and split into
//     two fp16 parts (hi, and lo = the rest), hi in output columns 0-7 and lo
//     in 8-15, so the split costs no extra MFMA and each part sums on its
//     own; products of fp16 parts and fp16 values are exact in fp32.  The
//     value rows, loaded as 16-byte pieces with the keys so that their
//     latency hides behind the logits, are transposed in registers (8x8
//     blocks of 16-bit elements) and through LDS to tokens x channels; the
//     chunk's sum is added into the rescaled running output.  16 heads:
//     lane l owns output channels D/64*l .., reads each token's weights from
//     LDS (broadcast) and sums on the VALU.
// The 8 waves' partial results are merged through LDS at the end.  With a
// workspace and few rows (decode), a row is split over several workgroups
// (chunks dealt round-robin to all their waves) whose partial results a
// second kernel merges.  Every sum is a chain of at most 64 + (chunks)
// terms, which the oracle's bound assumes.
#include "qsa_internal.h"

#include <math.h>

namespace qsa {
namespace {

constexpr int kAttnWaves = 8;
constexpr int kChunk = 64;

struct AttnArgs {
    const uint16_t *q16;
    int64_t qts;
    const uint16_t *k_tok, *v_tok;
    int64_t kvts;
    const int32_t *ids;
    int64_t ld_ids;
    float *out;
    int64_t ots;
    int32_t G, nq, H;
    int64_t n_kv, nb;
    int32_t bs, k;
    float scale;
    int32_t splits;   // workgroups per row; > 1: partial results go to ws
    float *ws;        // [row][split][H][2 + D]: maximum, denominator, numerator
};

__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// The weights enter the matrix cores scaled by 2^14 (exact: p <= 1, so p'
// <= 16384, inside fp16's range) and split into two fp16 parts, hi =
// fp16(p') and lo = fp16(p' - hi): hi + lo is within 2^-22 of p' relative,
// or 2^-25 absolute where lo falls below fp16's normal range (2^-39 in
// units of p).  Every product of a part and a value is exact in fp32.
constexpr float kWeightScale = 16384.0f;
constexpr float kWeightUnscale = 1.0f / 16384.0f;

// Halves e of eight registers (e = 0..7 over a uint4) as one uint4: the
// 8x8 transpose of 16-bit elements held by one lane, one output at a time.
__device__ __forceinline__ uint4 column_of(const uint4 (&x)[8], int e) {
    uint32_t w[8];
    #pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t v = e < 2 ? x[j].x : e < 4 ? x[j].y : e < 6 ? x[j].z : x[j].w;
        w[j] = (e & 1) ? v >> 16 : v & 0xffffu;
    }
    return make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                      w[6] | (w[7] << 16));
}

// The value of the lane 32 away (lanes 0-31 <-> 32-63).
__device__ __forceinline__ float swap32(float v, int lane) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, static_cast<uint32_t>((lane & 32) ? r[0] : r[1]));
}

// Orders one wave's LDS writes before its later reads (and reads before
// later writes) where lanes read what other lanes wrote: the compiler may
// otherwise move a lane's read above a write to another address of its own,
// which another lane's read depends on.
__device__ __forceinline__ void lds_wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Exclusive prefix sum of x over the wave's lanes, and the total.
__device__ __forceinline__ int lane_excl_scan(int x, int lane, int *total) {
    int v = x;
    #pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(v, d);
        if (lane >= d) v += y;
    }
    *total = __shfl(v, 63);
    return v - x;
}

// HM: heads per row rounded up to a power of two (1, 2, 4, 8, 16).  Heads
// past H carry zero queries: their logits and sums are computed and never
// stored, so every per-head loop is unrolled without branches and the
// per-head state stays in registers.
template <int D, int HM>
__global__ __launch_bounds__(64 * kAttnWaves) void attention_kernel(AttnArgs a) {
    constexpr int CPL = D / 64;   // output channels per lane (1 or 2)
    constexpr int KS = D / 16;    // K-steps of v_mfma_f32_32x32x16_f16
    // Up to 8 heads: the weighted values on the matrix cores
    // (v_mfma_f32_16x16x32_f16, A = the values transposed through LDS, B =
    // the weights' two fp16 parts, one head per column: hi in columns 0-7, lo
    // in 8-15).  16 heads: on the VALU, value rows in batches of VB.
    constexpr bool PVM = HM <= 8;
    constexpr int VB = 16;
    constexpr int LPR = D / 8;            // lanes per value row (16-byte pieces)
    constexpr int TPP = 8 * (64 / LPR);   // tokens per pass through vt: 32 or 64
    constexpr int NPASS = kChunk / TPP;
    constexpr int CB = TPP / 8;           // 8-token blocks of a vt row
    constexpr int NDB = D / 16;           // 16-channel blocks of the output
    __shared__ uint4 qh[HM][D / 8];                       // the row's queries, fp16 bits
    __shared__ float ps[PVM ? 1 : kAttnWaves][PVM ? 1 : kChunk][HM];   // weights (VALU path)
    // MFMA path, per wave: the chunk's weight parts [column][8-token block]
    // and one pass of values transposed [channel][8-token block], 8 fp16 per
    // uint4, the block index XORed with a function of the row so that the
    // fragment reads and the transposed writes spread over the banks
    __shared__ uint4 pw[PVM ? kAttnWaves : 1][PVM ? 16 * 8 : 1];
    __shared__ uint4 vt[PVM ? kAttnWaves : 1][PVM ? D * CB : 1];
    __shared__ float red_m[kAttnWaves][HM], red_l[kAttnWaves][HM];
    __shared__ float red_o[kAttnWaves][HM][D];

    const int H = a.H;
    const int64_t row = blockIdx.x / a.splits;      // r = g * nq + t
    const int split = static_cast<int>(blockIdx.x % a.splits);
    const int64_t g = row / a.nq, t = row % a.nq;
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;

    // queries of this row, fp16 bits, into LDS (zero past H)
    uint16_t *qh16 = reinterpret_cast<uint16_t *>(&qh[0][0]);
    for (int e = threadIdx.x; e < HM * D; e += 64 * kAttnWaves) {
        const int h = e / D, i = e % D;
        qh16[e] = h < H ? a.q16[t * a.qts + (g * H + h) * D + i] : static_cast<uint16_t>(0);
    }
    __syncthreads();

    // The logits of a 32-token tile for every head are one MFMA chain:
    // A = the tile's keys (token l%32, channels 16s + 8*(l/32) .. +7 in lane
    // l), B = the queries transposed (head l%32, the same channels), so lane
    // l receives head l%32's logits of tokens 8*(r/4) + 4*(l/32) + r%4,
    // r = 0..15.  fp16 products are exact and the sums fp32.
    const int hq = lane & 31, kc = lane >> 5;
    half8 qb[KS];
    #pragma unroll
    for (int s = 0; s < KS; ++s)
        qb[s] = hq < HM ? __builtin_bit_cast(half8, qh[hq][2 * s + kc]) : half8{};

    // running maximum and denominator of head hq (lanes hq and hq + 32 hold
    // the same), and the running output of every head for this lane's
    // channels CPL*lane ..
    float mh = -INFINITY, lh = 0.0f;
    float acc[PVM ? 1 : HM][CPL];
    #pragma unroll
    for (int h = 0; h < (PVM ? 1 : HM); ++h) {
        #pragma unroll
        for (int c = 0; c < CPL; ++c) acc[h][c] = 0.0f;
    }
    // MFMA path: lane l holds output column l%16 (head l%16's hi sum below
    // 8, head l%16 - 8's lo sum above) of channels 16*db + 4*(l/16) + r, all
    // scaled by 2^14
    floatx4 pacc[PVM ? NDB : 1];
    #pragma unroll
    for (int db = 0; db < (PVM ? NDB : 1); ++db) pacc[db] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (PVM) {
        // columns of heads past HM stay zero
        #pragma unroll
        for (int i = 0; i < 2; ++i) pw[w][lane + 64 * i] = make_uint4(0, 0, 0, 0);
    }
    // row d of vt holds its 8-token blocks in the order block ^ swz(d)
    auto swz = [](int d) { return ((d >> 1) ^ (d >> 3)) & (CB - 1); };

    const uint16_t *kg = a.k_tok + g * D;
    const uint16_t *vg = a.v_tok + g * D;
    // the row's ids, one per lane (k <= 64), read once.  Each lane counts
    // its slot's chunks of at most kChunk tokens (0 for an empty slot) and a
    // prefix sum gives the index of the slot's first chunk in slot order.
    // The chunks in that order are dealt round-robin to the kAttnWaves *
    // splits waves of the row: a wave visits only its own chunks, and finds
    // the slot of chunk ci as the last one whose first chunk is <= ci (a
    // ballot), its id and first chunk by v_readlane.  A walk over every slot
    // to find them (about 40 scalar instructions per slot, 64 slots) took
    // the decode step from 20.6 to 33.7 us and nq = 256 at 128K keys from
    // 97.9 to 109.1 us.
    const int idv = lane < a.k ? a.ids[row * a.ld_ids + lane] : -1;
    int nck = 0;
    if (idv >= 0 && idv < a.nb) {
        const int64_t len = min(static_cast<int64_t>(a.bs),
                                a.n_kv - static_cast<int64_t>(idv) * a.bs);
        nck = static_cast<int>((len + kChunk - 1) / kChunk);
    }
    int n_chunks;
    const int first = lane_excl_scan(nck, lane, &n_chunks);
    const int period = kAttnWaves * a.splits, mine = split * kAttnWaves + w;
    for (int ci = mine; ci < n_chunks; ci += period) {
        const uint64_t at_or_before = __ballot(nck > 0 && first <= ci);
        const int slot = 63 - __builtin_clzll(at_or_before);   // uniform
        const int b = __builtin_amdgcn_readlane(idv, slot);
        const int cf = __builtin_amdgcn_readlane(first, slot);
        const int64_t tb = static_cast<int64_t>(b) * a.bs;
        const int64_t te = min(tb + a.bs, a.n_kv);
        const int64_t c0 = tb + static_cast<int64_t>(ci - cf) * kChunk;
        const int n = static_cast<int>(min(static_cast<int64_t>(kChunk), te - c0));
        // 1. the chunk's loads, in flight together: the key fragments of
        //    its two 32-token tiles (tokens past the chunk read its first
        //    one; their logits are masked) and, with VB = 64, every
        //    token's values for this lane's channels (rows past the chunk
        //    repeat its last; their weights are 0 and their values are
        //    zeroed before use).  The values are not needed until the
        //    weights are known, so their latency hides behind the logits.
        uint4 ka[2][KS];
        #pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const int tk = 32 * mt + hq;
            const uint16_t *kp = kg + (c0 + (tk < n ? tk : 0)) * a.kvts + 8 * kc;
            #pragma unroll
            for (int s = 0; s < KS; ++s) ka[mt][s] = *reinterpret_cast<const uint4 *>(kp + 16 * s);
        }
        uint32_t vw[PVM ? 1 : VB];
        uint4 vv[PVM ? NPASS : 1][8];
        // raw buffer loads over the chunk's value rows
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(vg + c0 * a.kvts), 0, 0x7fffffff, 0x00020000);
        const int rowb = static_cast<int>(a.kvts * 2);
        // VALU path: one lane offset (its channels) and a scalar row offset
        // per load, so the loads need no per-row vector address registers
        const int vlane = CPL * 2 * lane;
        auto vload = [&](int j) -> uint32_t {
            const int r = j < n ? j : n - 1;   // rows past the chunk repeat its last
            if constexpr (CPL == 2)
                return __builtin_amdgcn_raw_buffer_load_b32(vrs, vlane, r * rowb, 0);
            else
                return __builtin_amdgcn_raw_buffer_load_b16(vrs, vlane, r * rowb, 0);
        };
        // MFMA path: lane l loads channels 8*(l%LPR) .. +7 of the rows
        // pass*TPP + 8*(l/LPR) + j of a pass (rows past the chunk repeat its
        // last; they are zeroed before use)
        const int vq = lane / LPR;   // the lane's 8-token group of a pass
        auto vload_pass = [&](int ps_) __attribute__((always_inline)) {
            #pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tt = ps_ * TPP + 8 * vq + j;
                const int r = tt < n ? tt : n - 1;
                vv[ps_][j] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, 16 * (lane % LPR) + r * rowb, 0, 0));
            }
        };
        if constexpr (PVM) {
            // the first pass's values are issued with the keys (not needed
            // until the weights are known, their latency hides behind the
            // logits); a second pass's once the logits have freed the key
            // registers
            vload_pass(0);
            // keep the loads here: sunk towards their use they would wait
            // out their latency after the softmax
            __builtin_amdgcn_sched_barrier(0);
        }
        // 2. logits: two 32x32 tiles (tokens x heads)
        floatx16 sa[2];
        #pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            #pragma unroll
            for (int s = 0; s < KS; ++s)
                sa[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    __builtin_bit_cast(half8, ka[mt][s]), qb[s], s == 0 ? floatx16{} : sa[mt],
                    0, 0, 0);
        }
        if constexpr (PVM && NPASS > 1) {
            vload_pass(1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // 3. weights of head hq and its running state: the chunk's
        //    maximum over the lane's 32 tokens and its partner's, the
        //    weights, their sum; the weights go to LDS for the values
        float cmax = -INFINITY;
        #pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int tk = 32 * mt + 8 * (r >> 2) + 4 * kc + (r & 3);
                sa[mt][r] = tk < n ? sa[mt][r] * a.scale : -INFINITY;
                cmax = fmaxf(cmax, sa[mt][r]);
            }
        }
        cmax = fmaxf(cmax, swap32(cmax, lane));
        const float mn = fmaxf(mh, cmax);
        float csum = 0.0f;
        #pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            #pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                // tokens 8*rq + 4*kc .. +3 of tile mt: one 8-byte piece of
                // an 8-token block of the weight parts
                float pq[4];
                #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * rq + i;
                    const int tk = 32 * mt + 8 * rq + 4 * kc + i;
                    const float p = tk < n ? expf(sa[mt][r] - mn) : 0.0f;
                    csum += p;
                    pq[i] = p;
                    if constexpr (!PVM) {
                        if (hq < HM) ps[w][tk][hq] = p;
                    }
                }
                if constexpr (PVM) {
                    if (hq < HM) {
                        uint32_t hb[4], lb[4];
                        #pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float ps14 = pq[i] * kWeightScale;
                            const _Float16 hi = static_cast<_Float16>(ps14);
                            const _Float16 lo = static_cast<_Float16>(ps14 - static_cast<float>(hi));
                            hb[i] = __builtin_bit_cast(uint16_t, hi);
                            lb[i] = __builtin_bit_cast(uint16_t, lo);
                        }
                        const int tb = 4 * mt + rq;   // 8-token block of the chunk
                        uint2 *dh = reinterpret_cast<uint2 *>(&pw[w][hq * 8 + (tb ^ hq)]) + kc;
                        uint2 *dl = reinterpret_cast<uint2 *>(&pw[w][(8 + hq) * 8 + (tb ^ hq)]) + kc;
                        *dh = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                        *dl = make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
                    }
                }
            }
        }
        csum += swap32(csum, lane);
        const float alpha = expf(mh - mn);   // 0 on the first chunk (mh = -inf)
        lh = lh * alpha + csum;
        mh = mn;
        // every head's rescale for the output this lane holds
        if constexpr (PVM) {
            // column l%16 is head (l%16) & 7's, whose alpha lane l & 7 holds
            const float al = __shfl(alpha, lane & 7);
            #pragma unroll
            for (int db = 0; db < NDB; ++db) pacc[db] *= al;
        } else {
            #pragma unroll
            for (int h = 0; h < HM; ++h) {
                const float ah = __builtin_bit_cast(
                    float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
                #pragma unroll
                for (int c = 0; c < CPL; ++c) acc[h][c] *= ah;
            }
        }
        // 4. this chunk's weighted values, added into the running output
        if constexpr (PVM) {
            // Per pass of TPP tokens: the lane's value rows transposed in
            // registers (an 8x8 block of 16-bit elements: its 8 channels of
            // 8 tokens) and written to vt as one 8-token piece per channel;
            // then per 32-token K-step one MFMA per 16-channel block, A =
            // vt's rows (channel l%16 of the block, tokens 8*(l/16) ..), B =
            // the weight parts (column l%16, the same tokens).  The chunk's
            // sum starts from zero and is added into the rescaled running
            // output, as on the VALU path.  One wave's LDS operations run
            // in order, so vt is rewritten per pass with no barrier.
            floatx4 pcs[NDB];
            #pragma unroll
            for (int ps_ = 0; ps_ < NPASS; ++ps_) {
                #pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (ps_ * TPP + 8 * vq + j >= n) vv[ps_][j] = make_uint4(0, 0, 0, 0);
                }
                #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = 8 * (lane % LPR) + e;
                    vt[w][d * CB + (vq ^ swz(d))] = column_of(vv[ps_], e);
                }
                lds_wave_sync();   // vt (and the weight parts) written, then read
                #pragma unroll
                for (int ks = 0; ks < TPP / 32; ++ks) {
                    const int kb = ps_ * (TPP / 32) + ks;   // K-step of the chunk
                    const int col = lane & 15, tq = lane >> 4;
                    const int tbk = 4 * kb + tq;             // 8-token block of the chunk
                    const half8 bf = __builtin_bit_cast(half8, pw[w][col * 8 + (tbk ^ (col & 7))]);
                    #pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const int d = 16 * db + col;
                        const int cbk = 4 * ks + tq;         // 8-token block of the pass
                        const half8 af = __builtin_bit_cast(half8, vt[w][d * CB + (cbk ^ swz(d))]);
                        pcs[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            af, bf, kb == 0 ? floatx4{0.0f, 0.0f, 0.0f, 0.0f} : pcs[db], 0, 0, 0);
                    }
                }
                lds_wave_sync();   // read before the next pass's or chunk's writes
            }
            #pragma unroll
            for (int db = 0; db < NDB; ++db) pacc[db] += pcs[db];
        } else {
            // 4. this chunk's weighted values (lane l owns channels CPL*l..),
            //    added into the running output; token j's weights are
            //    ps[w][j][*], 0 past the chunk
            lds_wave_sync();   // the weights written, then read by every lane
            float cs[HM][CPL];
            #pragma unroll
            for (int h = 0; h < HM; ++h) {
                #pragma unroll
                for (int c = 0; c < CPL; ++c) cs[h][c] = 0.0f;
            }
            auto pv = [&](int j, uint32_t bits) __attribute__((always_inline)) {
                float v[CPL];
                v[0] = f16_to_f32(bits & 0xffffu);
                if constexpr (CPL == 2) v[1] = f16_to_f32(bits >> 16);
                #pragma unroll
                for (int c = 0; c < CPL; ++c) v[c] = j < n ? v[c] : 0.0f;   // no 0 * inf
                #pragma unroll
                for (int h = 0; h < HM; ++h) {
                    const float p = ps[w][j][h];
                    #pragma unroll
                    for (int c = 0; c < CPL; ++c) cs[h][c] = __builtin_fmaf(p, v[c], cs[h][c]);
                }
            };
            // value rows in batches of VB, every load of a batch in
            // flight before its adds
            for (int j0 = 0; j0 < n; j0 += VB) {
                #pragma unroll
                for (int jj = 0; jj < VB; ++jj) vw[jj] = vload(j0 + jj);
                #pragma unroll
                for (int jj = 0; jj < VB; ++jj) pv(j0 + jj, vw[jj]);
            }
            #pragma unroll
            for (int h = 0; h < HM; ++h) {
                #pragma unroll
                for (int c = 0; c < CPL; ++c) acc[h][c] += cs[h][c];
            }
            lds_wave_sync();   // read before the next chunk's writes
        }
    }

    // 5. merge the waves' partial results
    if (lane < HM) {
        red_m[w][lane] = mh;
        red_l[w][lane] = lh;
    }
    if constexpr (PVM) {
        // head h's output is its hi column (lane l, l%16 = h) plus its lo
        // column (lane l + 8), unscaled by 2^-14
        #pragma unroll
        for (int db = 0; db < NDB; ++db) {
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float lo = __shfl_down(pacc[db][r], 8);
                if ((lane & 15) < HM)
                    red_o[w][lane & 15][16 * db + 4 * (lane >> 4) + r] =
                        (pacc[db][r] + lo) * kWeightUnscale;
            }
        }
    } else {
        #pragma unroll
        for (int h = 0; h < HM; ++h) {
            #pragma unroll
            for (int c = 0; c < CPL; ++c) red_o[w][h][CPL * lane + c] = acc[h][c];
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < H * D; e += 64 * kAttnWaves) {
        const int h = e / D, i = e % D;
        float M = -INFINITY;
        #pragma unroll
        for (int v = 0; v < kAttnWaves; ++v) M = fmaxf(M, red_m[v][h]);
        float num = 0.0f, den = 0.0f;
        if (M != -INFINITY) {
            #pragma unroll
            for (int v = 0; v < kAttnWaves; ++v) {
                const float f = red_m[v][h] == -INFINITY ? 0.0f : expf(red_m[v][h] - M);
                num = __builtin_fmaf(red_o[v][h][i], f, num);
                den = __builtin_fmaf(red_l[v][h], f, den);
            }
        }
        if (a.splits == 1) {
            a.out[t * a.ots + (g * H + h) * D + i] = den > 0.0f ? num / den : 0.0f;
        } else {
            float *part = a.ws + (static_cast<int64_t>(blockIdx.x) * H + h) * (2 + D);
            if (i == 0) {
                part[0] = M;
                part[1] = den;
            }
            part[2 + i] = num;
        }
    }
}

// Rows split over several workgroups: combine their partial results.  One
// thread per output element (head h, channel i), rows of H*D elements over
// as many 256-thread workgroups as they need; the splits' maxima, then their
// denominators and numerators, are loaded eight splits at a time, all eight
// in flight together (a merge of up to 8 splits is two memory round trips).
constexpr int kMergeBatch = 8;

template <int D>
__global__ __launch_bounds__(256) void attention_merge_kernel(AttnArgs a) {
    const int H = a.H;
    const int per_row = (H * D + 255) / 256;
    const int64_t row = blockIdx.x / per_row;
    const int e = static_cast<int>(blockIdx.x % per_row) * 256 + static_cast<int>(threadIdx.x);
    if (e >= H * D) return;
    const int h = e / D, i = e % D;
    const int64_t g = row / a.nq, t = row % a.nq;
    const int64_t sstride = static_cast<int64_t>(H) * (2 + D);   // floats between splits
    const float *base = a.ws + row * a.splits * sstride + static_cast<int64_t>(h) * (2 + D);
    float M = -INFINITY;
    for (int sp0 = 0; sp0 < a.splits; sp0 += kMergeBatch) {
        float mv[kMergeBatch];
        #pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
            mv[u] = sp0 + u < a.splits ? base[(sp0 + u) * sstride] : -INFINITY;
        #pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) M = fmaxf(M, mv[u]);
    }
    float num = 0.0f, den = 0.0f;
    if (M != -INFINITY) {
        for (int sp0 = 0; sp0 < a.splits; sp0 += kMergeBatch) {
            float mv[kMergeBatch], lv[kMergeBatch], ov[kMergeBatch];
            #pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const bool in = sp0 + u < a.splits;
                const float *part = base + (in ? sp0 + u : 0) * sstride;
                mv[u] = in ? part[0] : -INFINITY;
                lv[u] = part[1];
                ov[u] = part[2 + i];
            }
            #pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                // splits with no chunk hold -inf and add nothing
                const float f = mv[u] == -INFINITY ? 0.0f : expf(mv[u] - M);
                num = __builtin_fmaf(ov[u], f, num);
                den = __builtin_fmaf(lv[u], f, den);
            }
        }
    }
    a.out[t * a.ots + (g * H + h) * D + i] = den > 0.0f ? num / den : 0.0f;
}

template <int D>
void (*pick_attention(int H))(AttnArgs) {
    if (H <= 1) return attention_kernel<D, 1>;
    if (H <= 2) return attention_kernel<D, 2>;
    if (H <= 4) return attention_kernel<D, 4>;
    if (H <= 8) return attention_kernel<D, 8>;
    return attention_kernel<D, 16>;
}

}  // namespace

hipError_t launch_attention(const uint16_t *q16, int64_t qts, const uint16_t *k_tok,
                            const uint16_t *v_tok, int64_t kvts, const int32_t *ids, int64_t ld_ids,
                            float *out, int64_t ots, int32_t G, int32_t nq, int32_t H, int32_t D,
                            int64_t n_kv, int32_t bs, int32_t k, float *ws, int64_t ws_floats,
                            hipStream_t s) {
    const int64_t rows = static_cast<int64_t>(G) * nq;
    if (rows <= 0) return hipSuccess;
    int64_t sp = ws ? attention_splits(rows, bs, k) : 1;
    const int64_t per_split = rows * H * (2 + D);
    if (sp > 1 && sp * per_split > ws_floats) sp = ws_floats / per_split;
    if (sp < 2) sp = 1;
    if (rows * sp > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    AttnArgs a{q16, qts, k_tok, v_tok, kvts, ids, ld_ids, out, ots, G, nq, H,
               n_kv, n_kv / bs + (n_kv % bs != 0), bs, k,
               static_cast<float>(1.0 / sqrt(static_cast<double>(D))),
               static_cast<int32_t>(sp), ws};
    void (*fn)(AttnArgs) = D == 128 ? pick_attention<128>(H) : pick_attention<64>(H);
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(rows * sp)), dim3(64 * kAttnWaves), 0, s, a);
    if (sp > 1) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        void (*mf)(AttnArgs) = D == 128 ? attention_merge_kernel<128> : attention_merge_kernel<64>;
        const int64_t per_row = (static_cast<int64_t>(H) * D + 255) / 256;
        if (rows * per_row > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(mf, dim3(static_cast<unsigned>(rows * per_row)), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace qsa
