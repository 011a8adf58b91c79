// step_f32.hip -- a whole fp32 block top-k sparse decode step in ONE
// kernel for steps whose per-pair bytes are small (a short context and a
// small budget: the tiny fp32 layer).  Each (sequence, KV head) pair runs
// on `nsplit` workgroups of 8 waves; every one of them
//
//   1. rebuilds the newest block's summary in LDS (fp64 mean in token
//      order, rounded to fp32; split 0 also writes it to S) with wave 0,
//      while all waves score the pair's other blocks against the group's
//      query sum (fp64, the per-lane math and butterfly of k_block_score,
//      so the scores are bit for bit those of the two-kernel step); wave 0
//      then scores the newest block from its LDS row.  The scores stay in
//      LDS and are counted into the select's exponent tables;
//   2. selects the top k blocks (select.h; split 0 writes idx and, if
//      asked, the scores);
//   3. attends over its share of the kept tokens (fp32 MFMA, 16 tokens per
//      chunk); with one split it merges its waves into the output, else it
//      writes a partial (o, m, l) and the pair's last split to arrive
//      combines the partials (the workspace's arrival word of the pair).
//
// The steps are those of BlockTopKAttention (skill summary "Kinetics:
// Memory-Aware Test-Time Scaling", Implementation) with KV blocks and a
// budget of k blocks (rebuttal "Kinetics: Rethinking Test-Time Scaling
// Law", Q4 "KV block size and grouping strategy").
//
// Why this shape: such a step moves about a megabyte, so its time is a
// chain of latencies, and one compute unit pulls only ~50 GB/s (its
// outstanding misses are bounded): one workgroup per pair spent 12-14 us
// reading 512 KiB of kept K/V.  Splitting the kept tokens over several
// workgroups spreads those bytes over as many compute units; repeating the
// pair's small scan and selection in every split costs less than handing
// scores between workgroups (no wait anywhere: the arrival count is the
// only exchange, and nobody waits on it).
#include "attn_impl.h"
#include "score_impl.h"

namespace kin {

constexpr int kStepF32MaxBlocks = 8192;
// per-pair bytes (summary rows + kept K and V rows) up to which the fp32
// step runs as this one kernel
constexpr size_t kStepF32MaxPairBytes = (size_t)1 << 20;
// kept-token chunks (16 tokens) each split attends: 4 (64 tokens, 64 KiB of
// K and V)
constexpr int kStepF32ChunksPerSplit = 4;

struct StepF32Extra {
    void *S;
    double *scores;  // may be null: the scores are then not written out
    int32_t *idx;
    int nb_cap;
};

template <int KPT>
__global__ __launch_bounds__(kStepThreads) void k_decode_step_f32(AttnArgs a, StepF32Extra x,
                                                                  uint64_t *ctrl) {
    constexpr int NT = kStepThreads, NW = NT / 64;
    __shared__ int32_t sel[kStepIdxCap];
    __shared__ SelectLds<KPT, NT> sl;
    __shared__ union {
        double sc[kStepF32MaxBlocks];
        MergeLds<NW> m;
    } u;
    __shared__ uint32_t row_lds[kHeadDim];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int split = blockIdx.x, pair = blockIdx.y;
    const int b = pair / a.hkv, g = pair % a.hkv;
    const int nb = a.nb;
    const size_t row0 = (size_t)pair * x.nb_cap;
    double *sc_out = x.scores && split == 0 ? x.scores + row0 : nullptr;
    auto emit = [&](int j, double v) {
        if (v == 0.0) v = 0.0;  // one zero: -0.0 becomes +0.0
        u.sc[j] = v;
        if (sc_out) sc_out[j] = v;  // scores are an optional output
        select_count(sl, v);
    };

    // the attention's query operand, loaded now so its round trip overlaps
    // the scoring
    f32x4 qf[8];
    load_q_f32(a, pair, qf);
    select_clear(sl);
    __syncthreads();

    // 1. scores.  Rows of blocks below the newest one, 16 per wave and
    // round (4 rows per 16-lane group load), two rounds in flight: round
    // it + 2's loads are issued as soon as round it's math has read its
    // registers; past the range a load re-reads the last scored row and
    // its score is dropped.  The newest row is never loaded here: wave 0
    // rewrites it during this phase.  The first two rounds' loads go out
    // before the query rows are summed (they do not need the sum), so
    // their round trips overlap the query's and the newest row's (a pair
    // of 256 blocks is two rounds: one round trip for the whole scan).
    const int sub = lane & 15, grp = lane >> 4;
    const int n_rows = nb - 1;
    constexpr int kRound = NW * 16;
    const int n_it = wave * 16 < n_rows ? (n_rows - wave * 16 + kRound - 1) / kRound : 0;
    auto load_round = [&](int it, u32x4 (&ra)[4], u32x4 (&rb)[4]) {
        const int j0 = wave * 16 + it * kRound;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            load_row_slice<KIN_F32>(x.S, row0 + min(j0 + 4 * v + grp, n_rows - 1), sub, ra[v],
                                    rb[v]);
    };
    u32x4 wa[2][4], wb[2][4];
    if (n_it > 0) load_round(0, wa[0], wb[0]);
    if (n_it > 1) load_round(1, wa[1], wb[1]);
    double qs[8];
    group_query_sum<KIN_F32>(a.q, b, g, a.hkv, a.gqa, sub, qs);
    if (wave == 0)
        newest_summary<KIN_F32>(a.K, split == 0 ? x.S : nullptr, pair, a.t_cap, x.nb_cap,
                                a.ctx_len, a.block, row_lds, lane);
    wave_lds_sync();  // wave 0's row_lds entries, read across its lanes below
    if (n_it > 0) {
        for (int it = 0; it < n_it; ++it) {
            const int cur = it & 1;
            double part[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) part[v] = slice_dot<KIN_F32>(qs, wa[cur][v], wb[cur][v]);
            // this round's registers are read: they take round it + 2
            if (it + 2 < n_it) load_round(it + 2, wa[cur], wb[cur]);
            const double xv = fold4(part, lane);
            const int slot = ((lane & 8) ? 2 : 0) + ((lane & 4) ? 1 : 0);
            const int j = wave * 16 + it * kRound + 4 * slot + grp;
            if ((lane & 3) == 0 && j < n_rows) emit(j, xv);
        }
    }
    if (wave == 0) {
        // the newest row (written to row_lds by this wave) in slot 0 of row
        // group 0, zero rows elsewhere: the butterfly every block goes through
        const u32x4 zero = {0u, 0u, 0u, 0u};
        u32x4 ra = zero, rb = zero;
        if (grp == 0) {
            const uint32_t *r = row_lds + 8 * sub;
            ra = u32x4{r[0], r[1], r[2], r[3]};
            rb = u32x4{r[4], r[5], r[6], r[7]};
        }
        double part[4];
        part[0] = slice_dot<KIN_F32>(qs, ra, rb);
        part[1] = part[2] = part[3] = slice_dot<KIN_F32>(qs, zero, zero);
        const double xv = fold4(part, lane);
        if (lane == 0) emit(nb - 1, xv);
    }
    __syncthreads();

    // 2. selection (the scores are dead afterwards: the merge reuses them)
    select_topk<KPT, NT, true>(u.sc, nb, a.k, sel, sl);
    __syncthreads();
    if (split == 0)
        for (int i = tid; i < a.k; i += NT) x.idx[(size_t)pair * a.k + i] = sel[i];

    // 3. attention over this split's kept tokens, then the merge of the 8
    // waves; with several splits, the pair's last one combines
    const int cps = (a.n_chunks + a.nsplit - 1) / a.nsplit;
    const int c_beg = split * cps;
    const int c_end = min(a.n_chunks, c_beg + cps);
    attend_f32<ListRuns, NW>(a, list_runs(a, pair, sel), qf, c_beg, c_end, wave, NW, wave, u.m);
    __syncthreads();
    if (a.nsplit == 1) {
        merge_waves_and_store<KIN_F32, NW>(a, u.m, pair, 0);
        return;
    }
    merge_waves_and_store<KIN_F32, NW, true>(a, u.m, pair, split);
    stores_complete();
    __shared__ uint32_t last;
    __syncthreads();
    if (threadIdx.x == 0) {
        // the word was zero on entry (left so by the previous call on this
        // workspace); the last arrival leaves it at zero again
        last = arrive_add(ctrl + pair) == (uint32_t)a.nsplit;
        if (last) st_agent(ctrl + pair, (uint64_t)0);
    }
    __syncthreads();
    if (last) combine_pair<KIN_F32, NT>(a, pair);
}

// splits per pair of the one-kernel fp32 step
static int step_f32_splits(const Geo &g, int k) {
    const int keff = k < g.nb ? k : g.nb;
    const int n_chunks = (keff * g.block + kChunkF32 - 1) / kChunkF32;
    int ns = (n_chunks + kStepF32ChunksPerSplit - 1) / kStepF32ChunksPerSplit;
    if (ns > 64) ns = 64;
    if (ns < 1 || g.pairs > kCtrlWords) ns = 1;
    return ns;
}

size_t step_f32_ws_bytes(const Geo &g, int k) { return ws_total(ws_for(g, step_f32_splits(g, k))); }

bool step_f32_single_kernel(const Geo &g, int k) {
    if (g.dtype != KIN_F32 || g.nb > kStepF32MaxBlocks || k > kStepIdxCap) return false;
    const size_t keff = (size_t)(k < g.nb ? k : g.nb);
    const size_t row = (size_t)kHeadDim * sizeof(float);
    return (size_t)g.nb * row + keff * g.block * row * 2 <= kStepF32MaxPairBytes;
}

hipError_t launch_decode_step_f32(const Geo &g, const void *q, const void *K, const void *V,
                                  void *S, double *scores, int k, int32_t *idx, void *out,
                                  void *ws, hipStream_t s) {
    AttnPlan p;
    const int keff = k < g.nb ? k : g.nb;
    p.n_tokens = keff * g.block;
    p.n_chunks = (p.n_tokens + kChunkF32 - 1) / kChunkF32;
    p.nsplit = step_f32_splits(g, k);
    p.fused = 1;
    p.ws_bytes = step_f32_ws_bytes(g, k);
    AttnArgs a;
    fill_args(a, g, p, q, K, V, nullptr, k, out, ws);
    const StepF32Extra x{S, scores, idx, g.nb_cap};
    // the pair's arrival word: the start of the workspace
    uint64_t *ctrl = p.nsplit > 1 ? static_cast<uint64_t *>(ws) : nullptr;
    const dim3 grid(p.nsplit, g.pairs);
#define KIN_F32_STEP(KPT) k_decode_step_f32<KPT><<<grid, kStepThreads, 0, s>>>(a, x, ctrl)
    switch (select_kpt(g.nb, kStepThreads)) {
    case 1: KIN_F32_STEP(1); break;
    case 2: KIN_F32_STEP(2); break;
    case 4: KIN_F32_STEP(4); break;
    case 8: KIN_F32_STEP(8); break;
    default: KIN_F32_STEP(16); break;
    }
#undef KIN_F32_STEP
    return hipGetLastError();
}

}  // namespace kin
