// tok.hip -- token-level top-k decode step: every token is its own block
// (block size 1), so the keys are their own representatives and no summary
// array exists.  Per (sequence, KV head) pair:
//
//   kernel 1 (score.hip, k_score_tiles): the group score of every key,
//            fp64, streamed straight from K in tiles spread over the chip;
//   kernel 2 (here): the k best tokens (select_stream.h, the scores read
//            from memory), then attention over those tokens' K/V (MFMA,
//            online softmax), split over several workgroups when there are
//            fewer pairs than CUs, the splits combined in-kernel.
//
// The method is TopK attention over single tokens, the variant the
// rebuttal "Kinetics: Rethinking Test-Time Scaling Law" (Q2) names next to
// Block-TopK; here it is the block method with blocks of one token: score
// = sum over the group's query heads of q_h . k_t, top k tokens with ties
// to the lower index, softmax(q . k / sqrt(d)) over the kept tokens.
#include "attn_impl.h"
#include "select_stream.h"

namespace kin {

template <int NT>
struct TokLds {
    int32_t sel[kTokIdxCap];
    union {
        StreamSelectLds<NT> s;
        MergeLds<NT / 64> m;
    } u;
};

__global__ __launch_bounds__(kStepThreads) void k_tok_select_attend(AttnArgs a,
                                                                   const double *__restrict__ scores,
                                                                   int n_cap, int32_t *idx_out,
                                                                   uint64_t *ctrl) {
    constexpr int NW = kStepThreads / 64;
    __shared__ TokLds<kStepThreads> lds;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x, pair = blockIdx.y;

    // every split of a pair repeats the selection (it ends with a barrier)
    select_stream<kStepThreads>(scores + (size_t)pair * n_cap, a.ctx_len, a.k, lds.sel, lds.u.s);
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

// Token geometry: block 1, one "block" per token.
static Geo tok_geo(const Geo &g) {
    Geo t = g;
    t.block = 1;
    t.nb = g.ctx_len;
    t.nb_cap = g.t_cap;
    return t;
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
    // split partials, one arrival word per pair, then the scores
    const size_t part = ns == 1 ? 0 : align256(ws_for(g, ns)) + (size_t)g.pairs * sizeof(uint64_t);
    p.ws_bytes = align256(part) + (size_t)g.pairs * g.t_cap * sizeof(double);
    return p;
}

hipError_t launch_tok_step(const Geo &g0, const void *q, const void *K, const void *V,
                           double *scores, int k, int32_t *idx, void *out, void *ws, int num_cu,
                           hipStream_t s) {
    const Geo g = tok_geo(g0);
    const AttnPlan p = plan_tok(g, k, num_cu);
    char *w = static_cast<char *>(ws);
    uint64_t *ctrl = p.nsplit > 1 ? reinterpret_cast<uint64_t *>(w + align256(ws_for(g, p.nsplit)))
                                  : nullptr;
    const size_t part = p.nsplit == 1 ? 0 : align256(ws_for(g, p.nsplit)) + g.pairs * sizeof(uint64_t);
    double *sc = scores ? scores : reinterpret_cast<double *>(w + align256(part));
    // kernel 1: the scores straight from K (the keys are the summaries)
    hipError_t e = launch_score_rows(g, q, K, sc, num_cu, ctrl, s);
    if (e != hipSuccess) return e;
    AttnArgs a;
    fill_args(a, g, p, q, K, V, nullptr, k, out, ws);
    const dim3 grid(p.nsplit, g.pairs);
    k_tok_select_attend<<<grid, kStepThreads, 0, s>>>(a, sc, g.t_cap, idx, ctrl);
    return hipGetLastError();
}

}  // namespace kin
