// step.hip -- a whole block top-k sparse decode step in ONE kernel, one
// workgroup per (sequence, KV head) pair (8 waves, or 4 when two pairs share
// a CU):
//
//   1. wave 0 rebuilds the summary of the newest block (fp64 mean in token
//      order, rounded to bf16) and writes it to S, while
//   2. all waves score every other block of the pair against the group's
//      query sum (fp64, the same per-lane math and butterfly as the
//      standalone scoring kernel); wave 0 then scores the newest block from
//      its new row; the scores stay in LDS (and are written out);
//   3. the workgroup selects the top k blocks from LDS (select.h; the
//      exponent count tables are filled while the scores are made);
//   4. the waves attend over the kept blocks' K/V (MFMA, online softmax)
//      and merge into the output.  The attention walks a few blocks
//      already certain to be kept first (their sign/exponent bin lies above
//      the k-th key's, known from the count tables before the mantissa
//      passes) and the rest of the kept list after them, and with a
//      contiguous cache each wave loads its first chunk from those blocks
//      while step 3 still runs (the idx output stays the ascending list; the
//      order depends only on the scores, so every cache mode sums alike).
//
// The steps follow the method of BlockTopKAttention (skill summary
// "Kinetics: Memory-Aware Test-Time Scaling", Implementation) with KV
// blocks and a budget of k blocks (rebuttal "Kinetics: Rethinking
// Test-Time Scaling Law", Q4 "KV block size and grouping strategy").
//
// Why one kernel: a step streams two equal halves (the summary scan and
// the kept K/V gather) separated by a short dependent selection.  Between
// two kernels the chip idles for the launch gap and both kernels pay a
// ramp; inside one workgroup the selection reads its scores straight from
// LDS.  With at least as many pairs as CUs every CU streams its own pair
// from start to end.  (Handing scores between workgroups inside one kernel
// would need device-scope release/acquire per workgroup, which costs far
// more on this chip than a kernel boundary; so a pair stays in one
// workgroup.)  With fewer pairs than CUs the two-kernel split path is used.
//
// The scoring phase keeps a ring of four 16-row batches (4 KiB each) in
// flight per wave while it folds the oldest one.
#include "attn_impl.h"
#include "scoring.h"

namespace kin {

constexpr int kStepMaxBlocks = 8192;  // fp64 scores of one pair in LDS

// Two shapes of the step workgroup: 8 waves with room for 8192 scores (one
// workgroup per CU), or 4 waves with room for 2048 scores and at most 256
// registers per lane, so that two workgroups share a CU and one's
// selection and merge overlap the other's streaming (batches with at least
// two pairs per CU).
constexpr int kStepSmallWaves = 4;
constexpr int kStepSmallBlocks = 2048;
constexpr int kStepSmallMaxBlock = NewestLds<kStepSmallWaves>::kMaxBlock;

struct StepExtra {
    void *S;
    double *scores;  // may be null: the scores are then not written out
    int32_t *idx;
    int nb_cap;
};

// MODE kPaged: K/V through the page table (the kept blocks' first rows are
// looked up once, after the selection); kShared: a shared prompt's blocks
// from its own arrays (and the samples of a prompt launched next to each
// other on one XCD); the sequences may differ in length either way
// (for_pair).  QUEST: S holds two rows per block (channel-wise minimum and
// maximum of its keys) and a block's score is the Quest bound (scoring.h).
// NW waves; MAXNB: scores held in LDS.
template <int KPT, int MODE, int NW, int MAXNB, bool QUEST>
__global__ __launch_bounds__(NW * 64, NW == kStepSmallWaves ? 2 : 1) void k_decode_step(
    AttnArgs a0, StepExtra x) {
    constexpr int NT = NW * 64;
    static_assert(NW == kStepSmallWaves || NewestLds<NW>::kMaxBlock >= 128, "every block size");
    static_assert(!QUEST || MODE == kContig, "Quest summaries: contiguous caches");
    __shared__ int32_t sel[kStepIdxCap];
    __shared__ union {
        SelectLds<KPT, NT> sl;
        int64_t selrow[kStepIdxCap];  // PAGED, after the selection
    } su;
    SelectLds<KPT, NT> &sl = su.sl;
    __shared__ union {
        double sc[MAXNB];
        MergeLds<NW> m;
    } u;
    // After the scoring, the newest-row rebuild's LDS holds the attention's
    // block order: the list, the blocks put first (a bit per block) and
    // per-wave counts.  kPre: their first chunks are loaded during the
    // selection (contiguous caches).
    constexpr bool kPre = MODE == kContig;
    struct OrderLds {
        int32_t att[kStepIdxCap];
        uint32_t picked[MAXNB / 32];
        uint32_t pcnt[(kStepIdxCap / NT) * NW];
    };
    __shared__ union {
        NewestLds<NW> nl;
        OrderLds o;
    } nu;
    NewestLds<NW> &nl = nu.nl;
    int32_t *att = nu.o.att;
    uint32_t *picked = nu.o.picked;
    uint32_t *pcnt = nu.o.pcnt;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = MODE == kShared ? shared_pair(a0, blockIdx.x, gridDim.x) : blockIdx.x;
    const AttnArgs a = for_pair(a0, pair);
    const size_t row0 = (size_t)pair * x.nb_cap;
    const int nb = a.nb;

    // 1+2. score every block (wave 0 rebuilds the newest block's summary
    // first); the scores go to LDS and into the select's exponent tables
    select_clear(sl);
    if (tid == 0) nl.ready = 0u;
    __syncthreads();
    double *sc_out = x.scores ? x.scores + row0 : nullptr;
    // every block kept and no scores wanted: only the newest block's summary
    // is rebuilt (the range then holds just that block)
    const int j_beg = (a.k >= nb && !sc_out) ? nb - 1 : 0;
    auto emit = [&](int j, double v) {
        u.sc[j] = v;
        if (sc_out) sc_out[j] = v;  // scores are an optional output
        select_count(sl, v);
    };
    score_blocks<NW, true, decltype(emit), QUEST, MODE == kShared>(a, x.S, x.nb_cap, pair, j_beg,
                                                                  nb, nl, emit);
    __syncthreads();

    // 3. selection (reads the scores from LDS; they are dead afterwards, so
    //    the merge area may reuse them).  Once the k-th key's bin is
    //    known, P blocks above it (P blocks hold the NW waves' first chunks)
    //    go to att[0, P); kPre: every wave starts loading its first chunk.
    const int lane = tid & 63;
    ChunkRegs pre;
    bool use_pre = false;  // att holds the order (uniform)
    int n_pre = 0;
    auto early = [&](const uint64_t (&key)[KPT], uint32_t bin) {
        {
            bool cert[KPT];
            uint32_t mine = 0;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                cert[e] = (e * NT + tid < nb) && (uint32_t)(key[e] >> 52) > bin;
                mine += (uint32_t)__popcll(__ballot(cert[e]));
            }
            if (lane == 0) pcnt[wave] = mine;
            for (int i = tid; i < (nb + 31) / 32; i += NT) picked[i] = 0u;
            __syncthreads();
            uint32_t total = 0, run = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const uint32_t c = pcnt[w];
                total += c;
                run += w < wave ? c : 0u;
            }
            const int P = (NW * kChunkBf16 + a.block - 1) >> a.block_shift;
            if (total >= (uint32_t)P) {  // uniform
#pragma unroll
                for (int e = 0; e < KPT; ++e) {
                    const uint64_t m = __ballot(cert[e]);
                    const uint32_t r = run + rank_below(m);
                    const int j = e * NT + tid;
                    if (cert[e] && r < (uint32_t)P) {
                        att[r] = j;
                        atomicOr(&picked[j >> 5], 1u << (j & 31));
                    }
                    run += (uint32_t)__popcll(m);
                }
                __syncthreads();
                if constexpr (kPre) {
                    const ListRuns head{(int64_t)pair * a.t_cap, att, P, nb, a.block,
                                        a.block_shift};
                    load_chunk(a, head, static_cast<const uint16_t *>(a.K),
                               static_cast<const uint16_t *>(a.V), wave, lane & 15, lane >> 4,
                               pre);
                }
                use_pre = true;
                n_pre = P;
            }
        }
    };
    select_topk<KPT, NT, true>(u.sc, nb, a.k, sel, sl, early);
    __syncthreads();
    for (int i = tid; i < a.k; i += NT) x.idx[(size_t)pair * a.k + i] = sel[i];
    {
        if (use_pre) {  // uniform
            // att[P, keff): the kept blocks not loaded early, ascending (an
            // ordered compaction of sel)
            const int keff = min(a.k, nb);
            for (int i0 = 0; i0 < keff; i0 += NT) {
                const int id = i0 + tid < keff ? sel[i0 + tid] : -1;
                const bool rest = id >= 0 && !((picked[id >> 5] >> (id & 31)) & 1u);
                const uint64_t m = __ballot(rest);
                if (lane == 0) pcnt[(i0 / NT) * NW + wave] = (uint32_t)__popcll(m);
            }
            __syncthreads();
            for (int i0 = 0; i0 < keff; i0 += NT) {
                const int r0 = i0 / NT;
                uint32_t off = (uint32_t)n_pre;
                for (int q = 0; q < r0 * NW + wave; ++q) off += pcnt[q];
                const int id = i0 + tid < keff ? sel[i0 + tid] : -1;
                const bool rest = id >= 0 && !((picked[id >> 5] >> (id & 31)) & 1u);
                const uint64_t m = __ballot(rest);
                if (rest) att[off + rank_below(m)] = id;
            }
            __syncthreads();
        }
    }
    const int32_t *order = use_pre ? att : sel;  // the attention's block list

    // 4. attention over the kept blocks, then the merge of the 8 waves
    if constexpr (MODE == kPaged) {
        // first row of every kept block (a block lies inside one page); the
        // select's LDS is dead now
        for (int i = tid; i < a.k; i += NT) {
            const int id = order[i];
            su.selrow[i] = id >= 0 && id < nb ? token_row(a, pair, id * a.block) : -1;
        }
        __syncthreads();
        const PagedRuns runs{order, su.selrow, token_row(a, pair, 0), a.k, nb, a.block,
                             a.block_shift};
        attend_bf16<PagedRuns, NW>(a, runs, pair, 0, a.n_chunks, wave, NW, wave, u.m);
    } else if constexpr (MODE == kShared) {
        attend_bf16<SharedRuns, NW>(a, shared_runs(a, pair, order), pair, 0, a.n_chunks, wave,
                                    NW, wave, u.m);
    } else if constexpr (kPre) {
        attend_bf16<ListRuns, NW, true>(a, list_runs(a, pair, order), pair, 0, a.n_chunks, wave,
                                        NW, wave, u.m, &pre, use_pre);
    } else {
        attend_bf16<ListRuns, NW>(a, list_runs(a, pair, sel), pair, 0, a.n_chunks, wave, NW,
                                  wave, u.m);
    }
    __syncthreads();
    merge_waves_and_store<KIN_BF16, NW>(a, u.m, pair, 0);
}

// the 4-wave shape: at least two pairs per CU, and the pair fits its LDS
static bool step_small(const Geo &g, int cu) {
    return g.pairs >= 2 * cu && g.nb <= kStepSmallBlocks && g.block <= kStepSmallMaxBlock;
}

bool step_single_kernel(const Geo &g, int k, int num_cu) {
    const int cu = num_cu > 0 ? num_cu : 256;
    return g.dtype == KIN_BF16 && g.nb <= kStepMaxBlocks && k <= kStepIdxCap && g.pairs >= cu;
}

template <int NW, int MAXNB, bool QUEST>
static void launch_shape(const Geo &g, const AttnArgs &a, const StepExtra &x, hipStream_t s) {
    constexpr int NT = NW * 64;
    const dim3 grid(g.pairs);
#define KIN_STEP(KPT)                                                                          \
    do {                                                                                       \
        if constexpr (QUEST)                                                                   \
            k_decode_step<KPT, kContig, NW, MAXNB, true><<<grid, NT, 0, s>>>(a, x);            \
        else if (g.pages)                                                                      \
            k_decode_step<KPT, kPaged, NW, MAXNB, false><<<grid, NT, 0, s>>>(a, x);            \
        else if (g.share_n)                                                                    \
            k_decode_step<KPT, kShared, NW, MAXNB, false><<<grid, NT, 0, s>>>(a, x);           \
        else                                                                                   \
            k_decode_step<KPT, kContig, NW, MAXNB, false><<<grid, NT, 0, s>>>(a, x);           \
    } while (0)
    switch (select_kpt(g.nb, NT)) {
    case 1: KIN_STEP(1); break;
    case 2: KIN_STEP(2); break;
    case 4: KIN_STEP(4); break;
    case 8: KIN_STEP(8); break;
    default:
        if constexpr (MAXNB / NT >= 16) KIN_STEP(16);
        break;
    }
#undef KIN_STEP
}

hipError_t launch_decode_step(const Geo &g, const void *q, const void *K, const void *V, void *S,
                              double *scores, int k, int32_t *idx, void *out, int num_cu,
                              hipStream_t s, bool quest) {
    AttnPlan p;
    const int keff = k < g.nb ? k : g.nb;
    p.n_tokens = keff * g.block;
    p.n_chunks = (p.n_tokens + kChunkBf16 - 1) / kChunkBf16;
    p.nsplit = 1;
    p.fused = 1;
    p.ws_bytes = 0;
    AttnArgs a;
    fill_args(a, g, p, q, K, V, nullptr, k, out, nullptr);
    const StepExtra x{S, scores, idx, g.nb_cap};
    const bool small = step_small(g, num_cu > 0 ? num_cu : 256);
    if (quest && small)
        launch_shape<kStepSmallWaves, kStepSmallBlocks, true>(g, a, x, s);
    else if (quest)
        launch_shape<kStepThreads / 64, kStepMaxBlocks, true>(g, a, x, s);
    else if (small)
        launch_shape<kStepSmallWaves, kStepSmallBlocks, false>(g, a, x, s);
    else
        launch_shape<kStepThreads / 64, kStepMaxBlocks, false>(g, a, x, s);
    return hipGetLastError();
}

}  // namespace kin
