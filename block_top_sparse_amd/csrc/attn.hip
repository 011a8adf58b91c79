// attn.hip -- K4/K6: split-KV decode attention over a token list, K5: the
// log-sum-exp combine of the splits, and the fused second half of a decode
// step (top-k selection followed by attention, one workgroup per pair).
//
// For every query head h of KV head g,
//     out_h = sum_t softmax_t(q_h . k_t / sqrt(d)) v_t
// over the tokens of the kept blocks (sparse, the attention step of
// BlockTopKAttention in the skill summary "Kinetics: Memory-Aware Test-Time
// Scaling", Implementation: everything outside the kept blocks is masked
// before the softmax, which equals leaving it out), or over every token in
// [0, ctx_len) (dense, the comparison of the rebuttal "Kinetics: Rethinking
// Test-Time Scaling Law", "W2 & Q2: Real-world latency benchmarks").
//
// A pair's token list is cut into fixed chunks; a workgroup takes a
// contiguous range of chunks ("split"), its waves take chunks round-robin
// and keep a running max / sum / output (online softmax, base 2).  The
// waves are merged through LDS in a fixed order; with more than one split
// per pair the workgroup writes an unnormalised partial (o, m, l) and K5
// merges them.
//
// bf16 path (MFMA, gfx950 v_mfma_f32_16x16x32_bf16), 32 tokens per chunk:
//   S^T[token][head] = K_chunk . Q^T   two 16-token tiles x 4 k-steps of 32
//                                      channels; the GQA group (<= 16 heads)
//                                      fills the 16 columns, unused ones are 0
//   O[head][chan]   += P . V_chunk     8 MFMAs over 16-channel tiles
// Lane l (j = l % 16, g = l / 16) loads K rows of tokens 16*tau + j (16 B
// slices at channel 32*kk + 8*g) and V rows of tokens 16*tau + 4*g + r,
// r = 0..3, channels 8j..8j+7 -- every V load instruction reads 4 whole
// 256 B rows.  The MFMA output leaves lane l holding the scores of head j
// for exactly the tokens whose V rows it loaded, so P needs no data
// movement; V's 8x8 (token x channel) register block is transposed with
// 16-bit permutes into the B operand, and output column j of tile n is
// channel 8j + n.  Softmax weights enter the MFMA as bf16; the running sum
// uses the same rounded weights, so the weights still sum to one.  Each
// wave loads chunk c + stride while it computes chunk c (two register
// buffers), so a wave always has one chunk (16 KiB) of loads in flight.
//
// fp32 path (MFMA, v_mfma_f32_16x16x4_f32), 16 tokens per chunk: the same
// two products with 4-channel k-steps, laid out so that every load reads
// contiguous row pieces and the weights again stay in the lanes that
// computed them (attn_impl.h); fp32 weights and accumulation.
#include "attn_impl.h"

namespace kin {

template <bool DENSE>
__global__ __launch_bounds__(kAttnThreads) void k_attn_bf16(AttnArgs a) {
    __shared__ MergeLds<4> sm;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x, pair = blockIdx.y;
    const int cps = (a.n_chunks + a.nsplit - 1) / a.nsplit;
    const int c_beg = split * cps;
    const int c_end = min(a.n_chunks, c_beg + cps);
    if (DENSE)
        attend_bf16<DenseRuns, 4>(a, dense_runs(a, pair), pair, c_beg, c_end, wave, 4, wave, sm);
    else
        attend_bf16<ListRuns, 4>(a, list_runs(a, pair, a.idx + (size_t)pair * a.k), pair, c_beg,
                                 c_end, wave, 4, wave, sm);
    __syncthreads();
    merge_waves_and_store<KIN_BF16, 4>(a, sm, pair, split);
}

template <bool DENSE>
__global__ __launch_bounds__(kAttnThreads) void k_attn_f32(AttnArgs a) {
    __shared__ MergeLds<4> sm;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int split = blockIdx.x, pair = blockIdx.y;
    const int cps = (a.n_chunks + a.nsplit - 1) / a.nsplit;
    const int c_beg = split * cps;
    const int c_end = min(a.n_chunks, c_beg + cps);
    f32x4 qf[8];
    load_q_f32(a, pair, qf);
    if (DENSE)
        attend_f32<DenseRuns, 4>(a, dense_runs(a, pair), qf, c_beg, c_end, wave, 4, wave, sm);
    else
        attend_f32<ListRuns, 4>(a, list_runs(a, pair, a.idx + (size_t)pair * a.k), qf, c_beg,
                                c_end, wave, 4, wave, sm);
    __syncthreads();
    merge_waves_and_store<KIN_F32, 4>(a, sm, pair, split);
}

// ---------------------------------------------------------------------------
// fused decode-step second half: select, then attend (one workgroup per
// (pair, split); every split of a pair repeats the same selection)
// ---------------------------------------------------------------------------

// cand (bf16, tile candidates): the pair's n_cand candidates, in block
// order, their scores at scores + pair * n_cand and their block numbers at
// cand + pair * n_cand; the selection keeps k of them (places ascending,
// ties to the lower place, hence the lower block) and turns the places into
// block numbers.  Otherwise scores holds every block's score (stride nb_cap).
template <int DT, int KPT, int MODE>
__global__ __launch_bounds__(kStepThreads) void k_select_attend(AttnArgs a0,
                                                                const double *__restrict__ scores,
                                                                int nb_cap, int32_t *idx_out,
                                                                uint64_t *ctrl, void *S_newest,
                                                                const int32_t *cand, int n_cand) {
    constexpr int NW = kStepThreads / 64;
    __shared__ int32_t sel[kStepIdxCap];
    __shared__ union {
        SelectLds<KPT, kStepThreads> s;
        MergeLds<NW> m;
    } u;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int pair, split;
    split_slot(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, gridDim.y, pair, split);
    const AttnArgs a = for_pair(a0, pair);  // this sequence's own length
    // fp32: the attention's query operand, loaded before the selection
    f32x4 qf32[8];
    if constexpr (DT == KIN_F32) load_q_f32(a, pair, qf32);
    select_clear(u.s);
    __syncthreads();
    if (cand) {
        select_topk<KPT, kStepThreads, false>(scores + (size_t)pair * n_cand, n_cand, a.k, sel,
                                              u.s);
        __syncthreads();
        // k < n_cand and at least k candidates are real blocks (every tile
        // hands over min(k, its blocks)): every kept place holds a block
        const int32_t *cp = cand + (size_t)pair * n_cand;
        for (int i = threadIdx.x; i < a.k; i += kStepThreads) sel[i] = cp[sel[i]];
    } else {
        select_topk<KPT, kStepThreads, false>(scores + (size_t)pair * nb_cap, a.nb, a.k, sel,
                                              u.s);
    }
    __syncthreads();
    if (split == 0)
        for (int i = threadIdx.x; i < a.k; i += kStepThreads) idx_out[(size_t)pair * a.k + i] = sel[i];
    __syncthreads();  // selection done: its LDS is free for the merge

    // a step that keeps every block: the newest summary row is rebuilt here
    // (by the wave with the fewest chunks), the step has no scoring half
    if (DT == KIN_BF16 && S_newest && split == 0 && wave == NW - 1)
        newest_row_bf16(a, S_newest, nb_cap, pair, threadIdx.x & 63);

    const int cps = (a.n_chunks + a.nsplit - 1) / a.nsplit;
    const int c_beg = split * cps;
    const int c_end = min(a.n_chunks, c_beg + cps);
    if constexpr (DT == KIN_BF16 && MODE == kPaged) {
        // first row of every kept block (a block lies inside one page)
        __shared__ int64_t selrow[kStepIdxCap];
        for (int i = threadIdx.x; i < a.k; i += kStepThreads) {
            const int id = sel[i];
            selrow[i] = id >= 0 && id < a.nb ? token_row(a, pair, id * a.block) : -1;
        }
        __syncthreads();
        const PagedRuns runs{sel, selrow, token_row(a, pair, 0), a.k, a.nb, a.block,
                             a.block_shift};
        attend_bf16<PagedRuns, NW>(a, runs, pair, c_beg, c_end, wave, NW, wave, u.m);
    } else if constexpr (DT == KIN_BF16 && MODE == kShared) {
        attend_bf16<SharedRuns, NW>(a, shared_runs(a, pair, sel), pair, c_beg, c_end, wave, NW,
                                    wave, u.m);
    } else if constexpr (DT == KIN_BF16) {
        attend_bf16<ListRuns, NW>(a, list_runs(a, pair, sel), pair, c_beg, c_end, wave, NW, wave,
                                  u.m);
    } else {
        attend_f32<ListRuns, NW>(a, list_runs(a, pair, sel), qf32, c_beg, c_end, wave, NW, wave,
                                 u.m);
    }
    __syncthreads();
    if (a.nsplit == 1) {
        merge_waves_and_store<DT, NW>(a, u.m, pair, split);
        return;
    }
    // this split's partial, then the pair's last split combines all of them
    merge_waves_and_store<DT, NW, true>(a, u.m, pair, split);
    stores_complete();
    __shared__ uint32_t last;
    __syncthreads();
    if (threadIdx.x == 0) {
        last = arrive_add(ctrl + pair) == (uint32_t)a.nsplit;
        // every split of the pair has arrived: the word is left at zero for
        // the next call (or graph replay) on this workspace
        if (last) st_agent(ctrl + pair, (uint64_t)0);
    }
    __syncthreads();
    if (last) combine_pair<DT, kStepThreads>(a, pair);
}

// ---------------------------------------------------------------------------
// K5: combine the splits of each (sequence, query head)
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(64) void k_combine(const float *__restrict__ ws_o,
                                                const float *__restrict__ ws_ml,
                                                void *__restrict__ out, int nsplit) {
    const size_t row = blockIdx.x;  // b * hq + h
    const int lane = threadIdx.x;   // channels 2*lane, 2*lane+1
    const float *ml = ws_ml + row * nsplit * 2;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float w = (M == -INFINITY) ? 0.f : exp2f(ml[2 * s] - M);
        L += w * ml[2 * s + 1];
        const float2 v = reinterpret_cast<const float2 *>(ws_o + (row * nsplit + s) * kHeadDim)[lane];
        o0 += w * v.x;
        o1 += w * v.y;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (DT == KIN_BF16) {
        static_cast<uint32_t *>(out)[row * (kHeadDim / 2) + lane] =
            f32_to_bf16_bits(o0 * inv) | (f32_to_bf16_bits(o1 * inv) << 16);
    } else {
        reinterpret_cast<float2 *>(out)[row * (kHeadDim / 2) + lane] = make_float2(o0 * inv, o1 * inv);
    }
}

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------

static int chunk_tokens(const Geo &g) { return g.dtype == KIN_BF16 ? kChunkBf16 : kChunkF32; }


AttnPlan plan_attention(const Geo &g, int k, bool dense, int num_cu) {
    AttnPlan p;
    const int keff = dense ? 0 : (k < g.nb ? k : g.nb);
    p.n_tokens = dense ? g.ctx_len : keff * g.block;
    p.n_chunks = (p.n_tokens + chunk_tokens(g) - 1) / chunk_tokens(g);
    // aim for ~2 workgroups per CU, but give every wave at least one chunk
    const int target = 2 * (num_cu > 0 ? num_cu : 256);
    int ns = (target + g.pairs - 1) / g.pairs;
    const int max_ns = p.n_chunks / 4;
    if (ns > max_ns) ns = max_ns;
    if (ns > 64) ns = 64;
    if (ns < 1) ns = 1;
    p.nsplit = ns;
    p.fused = 0;
    p.ws_bytes = ws_total(ws_for(g, ns));
    return p;
}

AttnPlan plan_step(const Geo &g, int k, int num_cu) {
    const int keff = k < g.nb ? k : g.nb;
    if (k > kStepIdxCap) return plan_attention(g, k, false, num_cu);
    AttnPlan p;
    p.n_tokens = keff * g.block;
    p.n_chunks = (p.n_tokens + chunk_tokens(g) - 1) / chunk_tokens(g);
    // one 8-wave workgroup per pair fills the chip once there are as many
    // pairs as CUs; below that, split the kept blocks (the selection is then
    // repeated by every split of a pair, and a combine pass follows)
    const int cu = num_cu > 0 ? num_cu : 256;
    int ns = (cu + g.pairs - 1) / g.pairs;
    const int max_ns = p.n_chunks / 8;
    if (ns > max_ns) ns = max_ns;
    if (ns > 64) ns = 64;
    // one arrival word per pair for the in-kernel combine
    if (ns < 1 || g.pairs > kCtrlWords) ns = 1;
    p.nsplit = ns;
    p.fused = 1;
    // the arrival words, then the split partials
    p.ws_bytes = ws_total(ws_for(g, ns));
    return p;
}

double *step_scores_in_ws(const Geo &g, const AttnPlan &p, void *ws) {
    return reinterpret_cast<double *>(ws_body(ws) + align256(ws_for(g, p.nsplit)));
}

// tile candidates: their scores, then (256-byte aligned) their block numbers
static size_t cand_idx_offset(const Geo &g, const TileCands &tc) {
    return align256((size_t)g.pairs * tc.n * sizeof(double));
}

int32_t *step_cands_in_ws(const Geo &g, const AttnPlan &p, const TileCands &tc, void *ws) {
    return reinterpret_cast<int32_t *>(reinterpret_cast<char *>(step_scores_in_ws(g, p, ws)) +
                                       cand_idx_offset(g, tc));
}

size_t step_ws_with_scores(const Geo &g, const AttnPlan &p, int k, int num_cu) {
    size_t area = (size_t)g.pairs * (size_t)g.nb_cap * sizeof(double);
    if (k > 0) {
        const TileCands tc = step_tile_cands(g, k, num_cu);
        if (tc.tiles) {
            const size_t c = cand_idx_offset(g, tc) + (size_t)g.pairs * tc.n * sizeof(int32_t);
            area = c > area ? c : area;
        }
    }
    return kCtrlBytes + align256(ws_for(g, p.nsplit)) + area;
}

static hipError_t launch_combine(const Geo &g, const AttnArgs &a, void *out, int nsplit,
                                 hipStream_t s) {
    if (g.dtype == KIN_BF16)
        k_combine<KIN_BF16><<<g.batch * g.hq, 64, 0, s>>>(a.ws_o, a.ws_ml, out, nsplit);
    else
        k_combine<KIN_F32><<<g.batch * g.hq, 64, 0, s>>>(a.ws_o, a.ws_ml, out, nsplit);
    return hipGetLastError();
}

hipError_t launch_attention(const Geo &g, const AttnPlan &p, const void *q, const void *K,
                            const void *V, const int32_t *idx, int k, void *out, void *ws,
                            hipStream_t s) {
    AttnArgs a;
    fill_args(a, g, p, q, K, V, idx, k, out, ws);
    const bool dense = idx == nullptr;
    dim3 grid(p.nsplit, g.pairs);
    if (g.dtype == KIN_BF16) {
        if (dense)
            k_attn_bf16<true><<<grid, kAttnThreads, 0, s>>>(a);
        else
            k_attn_bf16<false><<<grid, kAttnThreads, 0, s>>>(a);
    } else {
        if (dense)
            k_attn_f32<true><<<grid, kAttnThreads, 0, s>>>(a);
        else
            k_attn_f32<false><<<grid, kAttnThreads, 0, s>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    return launch_combine(g, a, out, p.nsplit, s);
}

template <int DT>
static void launch_sa(const Geo &g, const AttnArgs &a, dim3 grid, const double *scores,
                      int32_t *idx, uint64_t *ctrl, void *S_newest, hipStream_t s,
                      const int32_t *cand, int n_cand) {
#define KIN_SA_MODE(KPT, MODE)                                                                 \
    k_select_attend<DT, KPT, MODE><<<grid, kStepThreads, 0, s>>>(a, scores, g.nb_cap, idx, ctrl, \
                                                                 S_newest, cand, n_cand)
#define KIN_SA(KPT)                                                                            \
    (DT != KIN_BF16 ? KIN_SA_MODE(KPT, kContig)                                                \
     : g.pages      ? KIN_SA_MODE(KPT, (DT == KIN_BF16 ? kPaged : kContig))                    \
     : g.share_n    ? KIN_SA_MODE(KPT, (DT == KIN_BF16 ? kShared : kContig))                   \
                    : KIN_SA_MODE(KPT, kContig))
    switch (select_kpt(cand ? n_cand : g.nb, kStepThreads)) {
    case 1: KIN_SA(1); break;
    case 2: KIN_SA(2); break;
    case 4: KIN_SA(4); break;
    case 8: KIN_SA(8); break;
    case 16: KIN_SA(16); break;
    default: KIN_SA(32); break;
    }
#undef KIN_SA
#undef KIN_SA_MODE
}

// one arrival word per pair at the start of the workspace (combined in-kernel)
uint64_t *step_ctrl(const AttnPlan &p, void *ws) {
    if (!p.fused || p.nsplit <= 1) return nullptr;
    return static_cast<uint64_t *>(ws);
}

hipError_t launch_select_attend(const Geo &g, const AttnPlan &p, const void *q, const void *K,
                                const void *V, const double *scores, int k, int32_t *idx,
                                void *out, void *ws, hipStream_t s, void *S_newest,
                                const int32_t *cand, int n_cand) {
    if (!p.fused) {
        hipError_t e = launch_block_topk(g, scores, k, idx, s);
        if (e != hipSuccess) return e;
        return launch_attention(g, p, q, K, V, idx, k, out, ws, s);
    }
    AttnArgs a;
    fill_args(a, g, p, q, K, V, nullptr, k, out, ws);
    uint64_t *ctrl = step_ctrl(p, ws);
    dim3 grid(p.nsplit, g.pairs);
    if (g.dtype == KIN_BF16)
        launch_sa<KIN_BF16>(g, a, grid, scores, idx, ctrl, S_newest, s, cand, n_cand);
    else
        launch_sa<KIN_F32>(g, a, grid, scores, idx, ctrl, nullptr, s, nullptr, 0);
    return hipGetLastError();
}

}  // namespace kin
