// qsa_blockkeys.hip -- the block keys k_b that the scorer reads, built from
// the token keys of a KV cache: the step before the select phase.
//
// The pages index one key vector k_b per KV block (Strata pull request #228,
// part 1, score formula) without defining it.  The reading taken here: the
// mean of the block's token keys, per KV head and channel, rounded once to
// the nearest fp16 (ties to even); the partial last block averages its own
// tokens.
//
// Exactness: an fp16 value is an integer multiple of 2^-24 below 2^16 in
// magnitude, so a sum of up to 8192 of them is a multiple of 2^-24 below 2^29:
// exact in float64 in any order.  The mean N / len (N = sum * 2^24, an exact
// int64) is then rounded to the fp16 grid with integer arithmetic, so the
// result is the correctly rounded mean, independent of the summation order
// and of the block length.
//
// Mapping: one wave per (KV head, block).  A token row of one head is D fp16
// (16-byte chunks); lane l takes chunk l % (D/8) of every (64/(D/8))-th
// token, issues all its 16-byte loads of the block before it adds, and
// accumulates its 8 channels in float64.  The lanes that share a chunk are
// then added with lane swaps, and each of them rounds and stores its share
// of the chunk's 8 channels.
// HBM-bound: 2*D bytes read per token and head, 2*D written per block.
#include "qsa_internal.h"

namespace qsa {
namespace {

// fp16 bits nearest (ties to even) to num / den * 2^-24, for |num| < 2^53
// and 1 <= den <= 8192.
__device__ uint32_t round_ratio_f16(int64_t num, int64_t den) {
    const uint32_t sign = num < 0 ? 0x8000u : 0u;
    const uint64_t a = static_cast<uint64_t>(num < 0 ? -num : num);
    if (a == 0) return 0u;   // an exact zero mean is +0
    const uint64_t d = static_cast<uint64_t>(den);
    // fl = floor(log2(a / d))
    const int la = 63 - __builtin_clzll(a), ld = 63 - __builtin_clzll(d);
    int fl = la - ld;
    const bool ge = fl >= 0 ? a >= (d << fl) : (a << -fl) >= d;
    if (!ge) --fl;
    // the value a/d * 2^-24 lies in the binade [2^E, 2^(E+1)), E = fl - 24;
    // below 2^-14 the grid is the subnormal one, whose spacing 2^-24 is that
    // of the binade E = -14
    int E = fl - 24 < -14 ? -14 : fl - 24;
    const int s = E + 14;                  // log2 of the spacing, in units of 2^-24
    const uint64_t unit = d << s;          // < 2^13 * 2^29
    // q = floor(a / (d * 2^s)) = floor(floor(a / 2^s) / d).  The quotient is
    // below 2^11 (a grid point below 2^(E+1)), so a >> s < 2^11 * d <= 2^24:
    // a 32-bit division instead of a 64-bit one
    const uint32_t x = static_cast<uint32_t>(a >> s);
    uint64_t q = x / static_cast<uint32_t>(d);
    const uint64_t r = a - q * unit;
    if (2 * r > unit || (2 * r == unit && (q & 1))) ++q;
    if (q < 1024) return sign | static_cast<uint32_t>(q);   // subnormal
    if (q == 2048) {   // rounded up into the next binade
        q = 1024;
        ++E;
    }
    if (E > 15) return sign | 0x7c00u;
    return sign | static_cast<uint32_t>((E + 15) << 10) | static_cast<uint32_t>(q - 1024);
}

template <int D>
__global__ __launch_bounds__(256) void block_keys_kernel(const uint16_t *__restrict__ k_tok,
                                                         int64_t tok_stride,
                                                         uint16_t *__restrict__ kblk,
                                                         int64_t khs, int32_t G, int64_t nb,
                                                         int64_t n_kv, int32_t bs) {
    constexpr int LPT = D / 8;     // lanes per token row (16-byte chunks)
    constexpr int TPL = 64 / LPT;  // tokens per wave load
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (item >= static_cast<int64_t>(G) * nb) return;   // whole wave
    const int lane = threadIdx.x & 63;
    const int64_t g = item / nb, b = item % nb;
    const int64_t t0 = b * bs;
    const int len = static_cast<int>(min(static_cast<int64_t>(bs), n_kv - t0));
    const int c = lane % LPT, r = lane / LPT;
    const uint16_t *src = k_tok + g * D + 8 * c;

    double acc[8];
    #pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    // batches of 16 loads in flight, then their adds
    for (int j0 = 0; j0 < len; j0 += 16 * TPL) {
        uint4 v[16];
        #pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = j0 + u * TPL + r;
            v[u] = t < len ? *reinterpret_cast<const uint4 *>(src + (t0 + t) * tok_stride)
                           : make_uint4(0, 0, 0, 0);
        }
        #pragma unroll
        for (int u = 0; u < 16; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += static_cast<double>(static_cast<float>(
                    __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[e] & 0xffffu))));
                acc[2 * e + 1] += static_cast<double>(static_cast<float>(
                    __builtin_bit_cast(_Float16, static_cast<uint16_t>(w[e] >> 16))));
            }
        }
    }
    // add the TPL lanes that hold the same chunk (exact in any order); the
    // butterfly leaves the chunk's sums in each of its TPL lanes
    #pragma unroll
    for (int m = LPT; m < 64; m <<= 1) {
        #pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], m);
    }
    // the TPL lanes of a chunk share its 8 roundings: lane r rounds channels
    // CPL*r ... CPL*r + CPL - 1 of the chunk
    constexpr int CPL = 8 / TPL;
    uint32_t h[CPL];
    #pragma unroll
    for (int j = 0; j < CPL; ++j) {
        double v = acc[j];
        #pragma unroll
        for (int e = CPL + j; e < 8; e += CPL)
            if (r == e / CPL) v = acc[e];
        h[j] = round_ratio_f16(static_cast<int64_t>(v * 16777216.0), len);
    }
    uint16_t *dst = kblk + g * khs + b * D + 8 * c + CPL * r;
    if constexpr (CPL == 2)
        *reinterpret_cast<uint32_t *>(dst) = h[0] | (h[1] << 16);
    else
        *dst = static_cast<uint16_t>(h[0]);
}

}  // namespace

hipError_t launch_block_keys(const uint16_t *k_tok, int64_t tok_stride, uint16_t *kblk,
                             int64_t khs, int32_t G, int32_t D, int64_t n_kv, int32_t bs,
                             hipStream_t s) {
    const int64_t nb = n_kv / bs + (n_kv % bs != 0);
    const int64_t items = static_cast<int64_t>(G) * nb;
    if (items <= 0) return hipSuccess;
    const int64_t grid = (items + 3) / 4;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (D == 128)
        hipLaunchKernelGGL(block_keys_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           s, k_tok, tok_stride, kblk, khs, G, nb, n_kv, bs);
    else
        hipLaunchKernelGGL(block_keys_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                           s, k_tok, tok_stride, kblk, khs, G, nb, n_kv, bs);
    return hipGetLastError();
}

}  // namespace qsa
