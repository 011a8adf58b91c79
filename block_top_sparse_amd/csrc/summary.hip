// summary.hip -- K1: block summaries (mean key of each KV block).
//
// The block representative is the mean of the block's keys: for a single
// query q, q . mean(k) is the mean of the token scores q . k, which is how
// the skill summary page "Kinetics: Memory-Aware Test-Time Scaling"
// (Implementation, BlockTopKAttention) ranks a block ("mean score per
// block").  Keeping the mean key turns the per-step ranking into a scan of
// one row per block instead of one row per token.
//
// Exactness contract: every channel is summed in fp64 in ascending token
// order, divided by the block's valid-token count in fp64 (IEEE division),
// rounded fp64 -> fp32 by the hardware conversion (round to nearest even)
// and, for bf16 caches, fp32 -> bf16 (round to nearest even).  The result
// is therefore a fixed function of the stored keys.
//
// Launch: one wave per block, four blocks per 256-thread workgroup; lane l
// owns channels 2l and 2l+1, so one token row (128 channels) is one
// coalesced 256 B (bf16) or 512 B (fp32) wave load.
#include "attn_impl.h"

namespace kin {

template <int DT>
__global__ __launch_bounds__(256) void k_block_summary(const void *__restrict__ Kv,
                                                       void *__restrict__ Sv, int t_cap,
                                                       int nb_cap, int ctx_len, int block, int j0,
                                                       int nj) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int jj = blockIdx.x * 4 + wave;
    if (jj >= nj) return;
    const int j = j0 + jj;
    const size_t pair = blockIdx.y;
    const int t0 = j * block;
    const int n = min(block, ctx_len - t0);

    double s0 = 0.0, s1 = 0.0;
    if (DT == KIN_BF16) {
        const uint32_t *k = static_cast<const uint32_t *>(Kv) +
                            (pair * (size_t)t_cap + (size_t)t0) * (kHeadDim / 2) + lane;
#pragma unroll 8
        for (int t = 0; t < n; ++t) {
            const uint32_t w = k[(size_t)t * (kHeadDim / 2)];
            s0 += (double)bf16_lo(w);
            s1 += (double)bf16_hi(w);
        }
    } else {
        const float2 *k = static_cast<const float2 *>(Kv) +
                          (pair * (size_t)t_cap + (size_t)t0) * (kHeadDim / 2) + lane;
#pragma unroll 8
        for (int t = 0; t < n; ++t) {
            const float2 v = k[(size_t)t * (kHeadDim / 2)];
            s0 += (double)v.x;
            s1 += (double)v.y;
        }
    }
    const double cnt = (double)n;
    const float m0 = (float)(s0 / cnt), m1 = (float)(s1 / cnt);
    const size_t o = (pair * (size_t)nb_cap + (size_t)j) * (kHeadDim / 2) + lane;
    if (DT == KIN_BF16) {
        static_cast<uint32_t *>(Sv)[o] = f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
    } else {
        static_cast<float2 *>(Sv)[o] = make_float2(m0, m1);
    }
}

// Variable lengths / paged caches (bf16): blocks j0 + (4 * blockIdx.x +
// wave) that intersect [t_begin, t_end) inside the pair's own context; the
// same arithmetic as above, rows found through token_row (a block lies
// inside one page, so its rows are consecutive).
__global__ __launch_bounds__(256) void k_block_summary_paged(AttnArgs a0, void *__restrict__ Sv,
                                                             int nb_cap, int t_begin, int t_end,
                                                             int j0, int nj) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int jj = blockIdx.x * 4 + wave;
    if (jj >= nj) return;
    const int j = j0 + jj;
    const int pair = blockIdx.y;
    const AttnArgs a = for_pair(a0, pair);
    const int t0 = j * a.block;
    const int te = min(t_end, a.ctx_len);
    if (t0 >= te || t0 + a.block <= t_begin) return;  // outside this sequence's range
    const int n = min(a.block, a.ctx_len - t0);
    const uint32_t *k = static_cast<const uint32_t *>(a.K) + token_row(a, pair, t0) * (kHeadDim / 2) +
                        lane;
    double s0 = 0.0, s1 = 0.0;
#pragma unroll 8
    for (int t = 0; t < n; ++t) {
        const uint32_t w = k[(size_t)t * (kHeadDim / 2)];
        s0 += (double)bf16_lo(w);
        s1 += (double)bf16_hi(w);
    }
    const double cnt = (double)n;
    const float m0 = (float)(s0 / cnt), m1 = (float)(s1 / cnt);
    static_cast<uint32_t *>(Sv)[((size_t)pair * nb_cap + (size_t)j) * (kHeadDim / 2) + lane] =
        f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
}

hipError_t launch_block_summary_paged(const Geo &g, const void *K, void *S, int t_begin,
                                      int t_end, hipStream_t s) {
    const int te = t_end < g.ctx_len ? t_end : g.ctx_len;
    if (t_begin >= te) return hipSuccess;
    const int j0 = t_begin / g.block, nj = (te - 1) / g.block + 1 - j0;
    AttnPlan p{};
    p.nsplit = 1;
    AttnArgs a;
    fill_args(a, g, p, nullptr, K, nullptr, nullptr, 1, nullptr, nullptr);
    dim3 grid((nj + 3) / 4, g.pairs);
    k_block_summary_paged<<<grid, 256, 0, s>>>(a, S, g.nb_cap, t_begin, t_end, j0, nj);
    return hipGetLastError();
}

hipError_t launch_block_summary(const Geo &g, const void *K, void *S, int j0, int j1,
                                hipStream_t s) {
    const int nj = j1 - j0;
    if (nj <= 0) return hipSuccess;
    dim3 grid((nj + 3) / 4, g.pairs);
    if (g.dtype == KIN_BF16)
        k_block_summary<KIN_BF16><<<grid, 256, 0, s>>>(K, S, g.t_cap, g.nb_cap, g.ctx_len,
                                                       g.block, j0, nj);
    else
        k_block_summary<KIN_F32><<<grid, 256, 0, s>>>(K, S, g.t_cap, g.nb_cap, g.ctx_len,
                                                      g.block, j0, nj);
    return hipGetLastError();
}

}  // namespace kin
