// tok.hip -- token-level top-k decode step: every token is its own block
// (block size 1), so the keys are their own representatives and no summary
// array exists.  Per (sequence, KV head) pair:
//
//   kernel 1 (k_tok_score): the group score of every key, fp64, streamed
//            straight from K in tiles spread over the chip (the scoring loop
//            of scoring.h); the top 32 bits of each score's order key
//            written out, and each tile's sign/exponent counts;
//   kernel 2 (k_tok_select_attend): the k best tokens (select_key32.h over
//            those words, read from memory, low words recomputed from K
//            only where they decide), then attention over those tokens' K/V
//            (MFMA, online softmax), split over several workgroups when
//            there are fewer pairs than CUs, the splits combined in-kernel.
//
// With at least as many pairs as CUs, a context of at most 32768 tokens and
// at most 2048 kept, the whole step runs in one kernel (k_tok_step), one
// workgroup per pair: the scores' top words stay in LDS and nothing per
// token is written to memory (select_key32.h).
//
// The method is TopK attention over single tokens, the variant the
// rebuttal "Kinetics: Rethinking Test-Time Scaling Law" (Q2) names next to
// Block-TopK; here it is the block method with blocks of one token: score
// = sum over the group's query heads of q_h . k_t, top k tokens with ties
// to the lower index, softmax(q . k / sqrt(d)) over the kept tokens.
#include "attn_impl.h"
#include "scoring.h"
#include "select_key32.h"

namespace kin {

constexpr int kTokScoreThreads = 512;

// Kernel 1: the group score of every key of one tile of a pair's tokens;
// the top word of its order key written to `keys` ([pair][t_cap]), the
// score itself to `scores` when asked for, and the tile's sign/exponent
// counts written to `tables` ([pair][tile][kExpBins]).  Also clears the
// pair's arrival word for kernel 2's combine.
__global__ __launch_bounds__(kTokScoreThreads) void k_tok_score(AttnArgs a, uint32_t *keys,
                                                               double *scores, int tile_rows,
                                                               uint32_t *tables,
                                                               uint64_t *ctrl_zero) {
    constexpr int NW = kTokScoreThreads / 64;
    __shared__ NewestLds<NW> nl;  // not used: no summary to rebuild
    __shared__ uint32_t fine[4096];
    const int pair = blockIdx.y, tile = blockIdx.x;
    if (ctrl_zero && tile == 0 && threadIdx.x == 0) ctrl_zero[pair] = 0ull;
    for (int i = threadIdx.x; i < 4096; i += kTokScoreThreads) fine[i] = 0u;
    __syncthreads();
    const int j_beg = tile * tile_rows;
    const int j_end = min(a.ctx_len, j_beg + tile_rows);
    uint32_t *kp = keys + (size_t)pair * a.t_cap;
    double *sp = scores ? scores + (size_t)pair * a.t_cap : nullptr;
    // the scores of a pair fall into a few sign/exponent bins: one atomic per
    // distinct bin of the wave, not one per key
    if (j_beg < j_end)
        score_blocks<NW, false>(a, const_cast<void *>(a.K), a.t_cap, pair, j_beg, j_end, nl,
                                [&](int j, double v) {
            const uint32_t top = (uint32_t)(order_key(v) >> 32);
            kp[j] = top;
            count_wave_aggregated(fine, top >> 20, true);
            if (sp) sp[j] = v;  // scores are an optional output
        });
    __syncthreads();
    uint32_t *t = tables + ((size_t)pair * gridDim.x + tile) * kExpBins;
    for (int i = threadIdx.x; i < kExpBins; i += kTokScoreThreads) t[i] = fine[i];
}

template <int NT>
struct TokLds {
    int32_t sel[kTokIdxCap];
    uint32_t coarse[kExpBins / 16];
    union {
        uint32_t fine[kExpBins];           // the pair's sign/exponent counts
        Key32Scratch<NT, kTokMaxLen> s;    // once they have been read
        MergeLds<NT / 64> m;               // after the selection
    } u;
};

__global__ __launch_bounds__(kStepThreads) void k_tok_select_attend(AttnArgs a,
                                                                   const uint32_t *__restrict__ keys,
                                                                   int32_t *idx_out,
                                                                   uint64_t *ctrl,
                                                                   const uint32_t *tables,
                                                                   int ntables) {
    constexpr int NW = kStepThreads / 64;
    __shared__ TokLds<kStepThreads> lds;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int pair, split;
    split_slot(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, gridDim.y, pair, split);

    // the pair's counts: its tiles' tables summed (one table's bins of this
    // thread loaded together)
    constexpr int kBinsPerThread = kExpBins / kStepThreads;
    const uint32_t *tp = tables + (size_t)pair * ntables * kExpBins + threadIdx.x;
    uint32_t c[kBinsPerThread] = {};
    for (int t = 0; t < ntables; ++t) {
        uint32_t v[kBinsPerThread];
#pragma unroll
        for (int e = 0; e < kBinsPerThread; ++e) v[e] = tp[(size_t)t * kExpBins + e * kStepThreads];
#pragma unroll
        for (int e = 0; e < kBinsPerThread; ++e) c[e] += v[e];
    }
#pragma unroll
    for (int e = 0; e < kBinsPerThread; ++e) lds.u.fine[threadIdx.x + e * kStepThreads] = c[e];
    __syncthreads();
    // every split of a pair repeats the selection (it ends with a barrier)
    const int b = pair / a.hkv, g = pair % a.hkv;
    const uint16_t *row0 = static_cast<const uint16_t *>(a.K) + (size_t)pair * a.t_cap * kHeadDim;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((size_t)b * a.hkv * a.gqa + (size_t)g * a.gqa) * kHeadDim;
    select_key32<kStepThreads, kTokMaxLen, kKey32BatchMem>(keys + (size_t)pair * a.t_cap,
                                                           a.ctx_len, a.k, lds.sel, lds.u.fine,
                                                           lds.coarse, lds.u.s, row0, qp, a.gqa);
    if (split == 0)
        for (int i = threadIdx.x; i < a.k; i += kStepThreads)
            idx_out[(size_t)pair * a.k + i] = lds.sel[i];
    __syncthreads();  // the selection's LDS is free for the merge

    const int cps = (a.n_chunks + a.nsplit - 1) / a.nsplit;
    const int c_beg = split * cps;
    const int c_end = min(a.n_chunks, c_beg + cps);
    const TokenRuns runs{(int64_t)pair * a.t_cap, lds.sel, a.k, a.ctx_len};
    attend_bf16<TokenRuns, NW>(a, runs, pair, c_beg, c_end, wave, NW, wave, lds.u.m);
    __syncthreads();
    if (a.nsplit == 1) {
        merge_waves_and_store<KIN_BF16, NW>(a, lds.u.m, pair, split);
        return;
    }
    merge_waves_and_store<KIN_BF16, NW, true>(a, lds.u.m, pair, split);
    stores_complete();
    __shared__ uint32_t last;
    __syncthreads();
    // the arrival words were cleared by kernel 1
    if (threadIdx.x == 0) last = arrive_add(ctrl + pair) == (uint32_t)a.nsplit;
    __syncthreads();
    if (last) combine_pair<KIN_BF16, kStepThreads>(a, pair);
}

// The whole token-level step for one pair per workgroup: the score of every
// key (the streaming loop over K), its order key's top word kept in LDS and
// its sign/exponent counted; the selection from those words (low words
// recomputed only for keys that share the k-th key's top word); then the
// attention over the kept tokens and the merge of the waves.  The fp64
// scores are written only when asked for.
constexpr int kTokStepMaxLen = 32768;
constexpr int kTokStepMaxK = kStepIdxCap;

__global__ __launch_bounds__(kStepThreads) void k_tok_step(AttnArgs a, double *scores,
                                                          int32_t *idx_out) {
    constexpr int NW = kStepThreads / 64;
    __shared__ union {
        uint32_t key[kTokStepMaxLen];
        MergeLds<NW> m;  // after the selection
    } u;
    __shared__ union {
        uint32_t fine[kExpBins];
        Key32Scratch<kStepThreads, kTokStepMaxLen> s;  // once the table has been read
    } v;
    __shared__ int32_t sel[kTokStepMaxK];
    __shared__ uint32_t coarse[kExpBins / 16];
    __shared__ NewestLds<NW> nl;  // not used: no summary to rebuild
    const int pair = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int i = threadIdx.x; i < kExpBins; i += kStepThreads) v.fine[i] = 0u;
    __syncthreads();
    const int L = a.ctx_len;
    double *sp = scores ? scores + (size_t)pair * a.t_cap : nullptr;
    score_blocks<NW, false>(a, const_cast<void *>(a.K), a.t_cap, pair, 0, L, nl,
                            [&](int j, double x) {
        const uint32_t top = (uint32_t)(order_key(x) >> 32);
        u.key[j] = top;
        count_wave_aggregated(v.fine, top >> 20, true);
        if (sp) sp[j] = x;  // scores are an optional output
    });
    __syncthreads();
    const int b = pair / a.hkv, g = pair % a.hkv;
    const uint16_t *row0 = static_cast<const uint16_t *>(a.K) + (size_t)pair * a.t_cap * kHeadDim;
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((size_t)b * a.hkv * a.gqa + (size_t)g * a.gqa) * kHeadDim;
    select_key32<kStepThreads, kTokStepMaxLen, kKey32BatchLds>(u.key, L, a.k, sel, v.fine, coarse,
                                                               v.s, row0, qp, a.gqa);
    for (int i = threadIdx.x; i < a.k; i += kStepThreads) idx_out[(size_t)pair * a.k + i] = sel[i];
    // the keys are dead: the merge area overlays them
    const TokenRuns runs{(int64_t)pair * a.t_cap, sel, a.k, L};
    attend_bf16<TokenRuns, NW>(a, runs, pair, 0, a.n_chunks, wave, NW, wave, u.m);
    __syncthreads();
    merge_waves_and_store<KIN_BF16, NW>(a, u.m, pair, 0);
}

static bool tok_single_kernel(const Geo &g, int k, int num_cu) {
    const int cu = num_cu > 0 ? num_cu : 256;
    return g.pairs >= cu && g.ctx_len <= kTokStepMaxLen && k <= kTokStepMaxK;
}

// Token geometry: block 1, one "block" per token.
static Geo tok_geo(const Geo &g) {
    Geo t = g;
    t.block = 1;
    t.nb = g.ctx_len;
    t.nb_cap = g.t_cap;
    return t;
}

// Score tiles per pair: about one workgroup per CU, rows a multiple of one
// round of the 8 waves.
static void tok_tiles(const Geo &g, int num_cu, int &tiles, int &rows) {
    constexpr int kRound = (kTokScoreThreads / 64) * kScoreBatch;
    const int cu = num_cu > 0 ? num_cu : 256;
    tiles = g.pairs >= cu ? 1 : (cu + g.pairs - 1) / g.pairs;
    rows = (g.ctx_len + tiles - 1) / tiles;
    rows = (rows + kRound - 1) / kRound * kRound;
    tiles = (g.ctx_len + rows - 1) / rows;
}

// Workspace of the two-kernel token step: split partials, arrival words,
// the keys' top words, count tables (in that order, each 256-byte aligned).
struct TokWs {
    size_t ctrl, keys, tables, total;
};
static TokWs tok_ws(const Geo &g, int nsplit, int tiles) {
    TokWs w;
    w.ctrl = align256(ws_for(g, nsplit));
    w.keys = align256(w.ctrl + (nsplit > 1 ? (size_t)g.pairs * sizeof(uint64_t) : 0));
    w.tables = align256(w.keys + (size_t)g.pairs * g.t_cap * sizeof(uint32_t));
    w.total = w.tables + (size_t)g.pairs * tiles * kExpBins * sizeof(uint32_t);
    return w;
}

AttnPlan plan_tok(const Geo &g, int k, int num_cu) {
    const int keff = k < g.ctx_len ? k : g.ctx_len;
    AttnPlan p;
    p.n_tokens = keff;
    p.n_chunks = (keff + kChunkBf16 - 1) / kChunkBf16;
    const int cu = num_cu > 0 ? num_cu : 256;
    int ns = (cu + g.pairs - 1) / g.pairs;
    const int max_ns = p.n_chunks / 8;
    if (ns > max_ns) ns = max_ns;
    if (ns > 64) ns = 64;
    if (ns < 1) ns = 1;
    p.nsplit = ns;
    p.fused = 1;
    int tiles, rows;
    tok_tiles(g, num_cu, tiles, rows);
    p.ws_bytes = tok_ws(g, ns, tiles).total;
    return p;
}

hipError_t launch_tok_step(const Geo &g0, const void *q, const void *K, const void *V,
                           double *scores, int k, int32_t *idx, void *out, void *ws, int num_cu,
                           hipStream_t s) {
    const Geo g = tok_geo(g0);
    if (tok_single_kernel(g, k, num_cu)) {
        AttnPlan p{};
        p.n_tokens = k < g.ctx_len ? k : g.ctx_len;
        p.n_chunks = (p.n_tokens + kChunkBf16 - 1) / kChunkBf16;
        p.nsplit = 1;
        p.fused = 1;
        AttnArgs a;
        fill_args(a, g, p, q, K, V, nullptr, k, out, nullptr);
        k_tok_step<<<g.pairs, kStepThreads, 0, s>>>(a, scores, idx);
        return hipGetLastError();
    }
    const AttnPlan p = plan_tok(g, k, num_cu);
    int tiles, rows;
    tok_tiles(g, num_cu, tiles, rows);
    const TokWs wl = tok_ws(g, p.nsplit, tiles);
    char *w = static_cast<char *>(ws);
    uint64_t *ctrl = p.nsplit > 1 ? reinterpret_cast<uint64_t *>(w + wl.ctrl) : nullptr;
    uint32_t *keys = reinterpret_cast<uint32_t *>(w + wl.keys);
    uint32_t *tables = reinterpret_cast<uint32_t *>(w + wl.tables);
    AttnArgs a;
    fill_args(a, g, p, q, K, V, nullptr, k, out, ws);
    // kernel 1: the scores straight from K (the keys are the summaries)
    k_tok_score<<<dim3(tiles, g.pairs), kTokScoreThreads, 0, s>>>(a, keys, scores, rows, tables,
                                                                  ctrl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(p.nsplit, g.pairs);
    k_tok_select_attend<<<grid, kStepThreads, 0, s>>>(a, keys, idx, ctrl, tables, tiles);
    return hipGetLastError();
}

}  // namespace kin
