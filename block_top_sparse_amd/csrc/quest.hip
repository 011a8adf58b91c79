// quest.hip -- the Quest-style representative: each KV block is boxed by
// the channel-wise minimum and maximum of its keys, and ranked by the
// largest value q.k can take inside the box, summed over the GQA group's
// heads (the rebuttal "Kinetics: Rethinking Test-Time Scaling Law" names
// Quest as the second grouping strategy beside Block-TopK, Q4 "KV block
// size and grouping strategy"; the bound is the published Quest criterion).
//
//   k_quest_summary: the minimum and maximum rows of every block of a token
//                    range (one wave per block, strict comparisons in token
//                    order), into Sq [pair][nb_cap][2][d];
//   k_quest_tiles:   the decode step's first kernel: the newest block's two
//                    rows rebuilt and every block's bound (the scoring loop
//                    of scoring.h over the summary rows, P . max + N . min),
//                    in tiles spread over the chip;
// then the block method's second kernel (attn.hip, k_select_attend) keeps the
// k best blocks and attends over them.
#include "attn_impl.h"
#include "scoring.h"

namespace kin {

constexpr int kQuestThreads = 512;

__global__ __launch_bounds__(256) void k_quest_summary(const void *__restrict__ Kv,
                                                       void *__restrict__ Sv, int t_cap,
                                                       int nb_cap, int ctx_len, int block, int j0,
                                                       int nj) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int jj = blockIdx.x * 4 + wave;
    if (jj >= nj) return;
    const int j = j0 + jj;
    const int pair = blockIdx.y;
    const int t0 = j * block;
    const int n = min(block, ctx_len - t0);
    const uint32_t *k = static_cast<const uint32_t *>(Kv) +
                        ((size_t)pair * t_cap + t0) * (kHeadDim / 2) + lane;
    const uint32_t v0 = k[0];
    float lo0 = bf16_lo(v0), hi0 = lo0, lo1 = bf16_hi(v0), hi1 = lo1;
    uint32_t blo0 = v0 & 0xFFFFu, bhi0 = blo0, blo1 = v0 >> 16, bhi1 = blo1;
    for (int t = 1; t < n; ++t) {
        const uint32_t v = k[(size_t)t * (kHeadDim / 2)];
        const float x0 = bf16_lo(v), x1 = bf16_hi(v);
        if (x0 < lo0) { lo0 = x0; blo0 = v & 0xFFFFu; }
        if (x0 > hi0) { hi0 = x0; bhi0 = v & 0xFFFFu; }
        if (x1 < lo1) { lo1 = x1; blo1 = v >> 16; }
        if (x1 > hi1) { hi1 = x1; bhi1 = v >> 16; }
    }
    uint32_t *s = static_cast<uint32_t *>(Sv) + ((size_t)pair * nb_cap + j) * 2 * (kHeadDim / 2);
    s[lane] = blo0 | (blo1 << 16);
    s[kHeadDim / 2 + lane] = bhi0 | (bhi1 << 16);
}

template <bool UPDATE>
__global__ __launch_bounds__(kQuestThreads) void k_quest_tiles(AttnArgs a, void *Sq,
                                                              double *scores, int nb_cap,
                                                              int tile_rows, uint64_t *ctrl_zero) {
    constexpr int NW = kQuestThreads / 64;
    static_assert(NewestLds<NW>::kMaxBlock >= 128, "every block size");
    __shared__ NewestLds<NW> nl;
    const int pair = blockIdx.y;
    if (ctrl_zero && blockIdx.x == 0 && threadIdx.x == 0) ctrl_zero[pair] = 0ull;
    const int nb = a.nb;
    const int j_beg = blockIdx.x * tile_rows;
    if (j_beg >= nb) return;
    const int j_end = min(nb, j_beg + tile_rows);
    double *sp = scores + (size_t)pair * nb_cap;
    auto emit = [&](int j, double v) { sp[j] = v; };
    if (UPDATE && j_end == nb) {
        if (threadIdx.x == 0) nl.ready = 0u;
        __syncthreads();
        score_blocks<NW, true, decltype(emit), true>(a, Sq, nb_cap, pair, j_beg, nb, nl, emit);
    } else {
        score_blocks<NW, false, decltype(emit), true>(a, Sq, nb_cap, pair, j_beg, j_end, nl,
                                                      emit);
    }
}

hipError_t launch_quest_summary(const Geo &g, const void *K, void *Sq, int j0, int j1,
                                hipStream_t s) {
    const int nj = j1 - j0;
    if (nj <= 0) return hipSuccess;
    dim3 grid((nj + 3) / 4, g.pairs);
    k_quest_summary<<<grid, 256, 0, s>>>(K, Sq, g.t_cap, g.nb_cap, g.ctx_len, g.block, j0, nj);
    return hipGetLastError();
}

hipError_t launch_quest_score(const Geo &g, const void *q, const void *K, void *Sq,
                              double *scores, int num_cu, uint64_t *ctrl_zero, bool update,
                              hipStream_t s) {
    AttnPlan p{};
    p.nsplit = 1;
    AttnArgs a;
    fill_args(a, g, p, q, K, nullptr, nullptr, 1, nullptr, nullptr);
    // tiles of whole rounds of the 8 waves (a round covers kRound rows, two
    // rows per block)
    constexpr int kRoundBlocks = (kQuestThreads / 64) * kScoreBatch / 2;
    const int cu = num_cu > 0 ? num_cu : 256;
    const int tiles = g.pairs >= cu ? 1 : (cu + g.pairs - 1) / g.pairs;
    int rows = (g.nb + tiles - 1) / tiles;
    rows = (rows + kRoundBlocks - 1) / kRoundBlocks * kRoundBlocks;
    const dim3 grid((g.nb + rows - 1) / rows, g.pairs);
    if (update)
        k_quest_tiles<true><<<grid, kQuestThreads, 0, s>>>(a, Sq, scores, g.nb_cap, rows,
                                                           ctrl_zero);
    else
        k_quest_tiles<false><<<grid, kQuestThreads, 0, s>>>(a, Sq, scores, g.nb_cap, rows,
                                                            ctrl_zero);
    return hipGetLastError();
}

}  // namespace kin
