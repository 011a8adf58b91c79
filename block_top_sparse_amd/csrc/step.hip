// step.hip -- a whole block top-k sparse decode step in ONE kernel, one
// 512-thread workgroup per (sequence, KV head) pair:
//
//   1. wave 0 rebuilds the summary of the newest block (fp64 mean in token
//      order, rounded to bf16) and writes it to S, while
//   2. all 8 waves score every other block of the pair against the group's
//      query sum (fp64, the same per-lane math and butterfly as the
//      standalone scoring kernel); wave 0 then scores the newest block from
//      its new row; the scores stay in LDS (and are written out);
//   3. the workgroup selects the top k blocks from LDS (select.h);
//   4. the 8 waves attend over the kept blocks' K/V (MFMA, online softmax)
//      and merge into the output.
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
// The scoring phase double-buffers its row loads: each wave keeps one
// 64-block batch (16 KiB) in flight while it folds the previous one.
#include "attn_impl.h"
#include "score_impl.h"

namespace kin {

constexpr int kStepMaxBlocks = 8192;  // fp64 scores of one pair in LDS

struct StepExtra {
    void *S;
    double *scores;
    int32_t *idx;
    int nb_cap;
};

// Load this wave's 64-block batch starting at j0 (16 lanes per row, 4 rows
// per load, 4 tiles); rows past nb re-read row nb - 1 (never used).
__device__ __forceinline__ void load_batch(const uint16_t *S, size_t row0, int j0, int nb,
                                           int sub, int grp, u32x4 (&w)[4][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = min(j0 + 16 * t + 4 * u + grp, nb - 1);
            w[t][u] = ld_nt16(S + (row0 + j) * kHeadDim + 8 * sub);
        }
}

__device__ __forceinline__ void score_batch(const double (&qs)[8], const u32x4 (&w)[4][4], int j0,
                                            int nb, int lane, int grp, double *sc_lds,
                                            double *sc_out) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        double part[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) part[u] = slice_dot<KIN_BF16>(qs, w[t][u], zero);
        double x = fold4(part, lane);
        const int u = ((lane & 8) ? 2 : 0) + ((lane & 4) ? 1 : 0);
        const int j = j0 + 16 * t + 4 * u + grp;
        if ((lane & 3) == 0 && j < nb - 1) {  // the newest block is scored apart
            if (x == 0.0) x = 0.0;  // one zero: -0.0 becomes +0.0
            sc_lds[j] = x;
            sc_out[j] = x;
        }
    }
}

template <int KPT>
__global__ __launch_bounds__(kStepThreads) void k_decode_step(AttnArgs a, StepExtra x) {
    constexpr int NW = kStepThreads / 64;
    __shared__ int32_t sel[kStepIdxCap];
    __shared__ SelectLds<KPT, kStepThreads> sl;
    __shared__ union {
        double sc[kStepMaxBlocks];
        MergeLds<NW> m;
    } u;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = blockIdx.x;
    const int b = pair / a.hkv, g = pair % a.hkv;
    const size_t row0 = (size_t)pair * x.nb_cap;
    const int nb = a.nb;

    // 1+2. wave 0 rebuilds the newest block's summary while the other waves
    // start scoring; every wave skips the newest block in its batches, and
    // wave 0 scores it last from the LDS copy of the new row (same math).
    {
        __shared__ uint32_t newest_row[kHeadDim];
        const int sub = lane & 15, grp = lane >> 4;
        if (wave == 0)
            newest_summary<KIN_BF16>(a.K, x.S, pair, a.t_cap, x.nb_cap, a.ctx_len, a.block,
                                     newest_row, lane);
        double qs[8];
        group_query_sum<KIN_BF16>(a.q, b, g, a.hkv, a.gqa, sub, qs);
        const uint16_t *S = static_cast<const uint16_t *>(x.S);
        double *sc_out = x.scores + row0;
        constexpr int kBatch = 64;  // blocks per wave per batch
        const int jw = wave * kBatch;
        const int n = jw < nb ? (nb - jw + NW * kBatch - 1) / (NW * kBatch) : 0;
        u32x4 wa[4][4], wb[4][4];
        if (n > 0) {
            // the prefetch inside the loop is unconditional (tail peeled), so
            // the wait before a batch's math covers only that batch's loads
            load_batch(S, row0, jw, nb, sub, grp, wa);
            int i = 0;
            for (; i + 2 < n; i += 2) {
                load_batch(S, row0, jw + (i + 1) * NW * kBatch, nb, sub, grp, wb);
                score_batch(qs, wa, jw + i * NW * kBatch, nb, lane, grp, u.sc, sc_out);
                load_batch(S, row0, jw + (i + 2) * NW * kBatch, nb, sub, grp, wa);
                score_batch(qs, wb, jw + (i + 1) * NW * kBatch, nb, lane, grp, u.sc, sc_out);
            }
            if (n - i == 2) {
                load_batch(S, row0, jw + (i + 1) * NW * kBatch, nb, sub, grp, wb);
                score_batch(qs, wa, jw + i * NW * kBatch, nb, lane, grp, u.sc, sc_out);
                score_batch(qs, wb, jw + (i + 1) * NW * kBatch, nb, lane, grp, u.sc, sc_out);
            } else {
                score_batch(qs, wa, jw + i * NW * kBatch, nb, lane, grp, u.sc, sc_out);
            }
        }
        if (wave == 0) {
            // the newest row in slot u = 0 of row group 0, zero rows elsewhere
            const u32x4 zero = {0u, 0u, 0u, 0u};
            u32x4 r = zero;
            if (grp == 0) {
                const uint32_t *p = newest_row + 4 * sub;
                r = u32x4{p[0], p[1], p[2], p[3]};
            }
            double part[4];
            part[0] = slice_dot<KIN_BF16>(qs, r, zero);
            part[1] = part[2] = part[3] = slice_dot<KIN_BF16>(qs, zero, zero);
            double v = fold4(part, lane);
            if (lane == 0) {
                if (v == 0.0) v = 0.0;
                u.sc[nb - 1] = v;
                sc_out[nb - 1] = v;
            }
        }
    }
    __syncthreads();

    // 3. selection (reads the scores from LDS; they are dead afterwards, so
    //    the merge area may reuse them)
    select_topk<KPT, kStepThreads>(u.sc, nb, a.k, sel, sl);
    __syncthreads();
    for (int i = tid; i < a.k; i += kStepThreads) x.idx[(size_t)pair * a.k + i] = sel[i];

    // 4. attention over the kept blocks, then the merge of the 8 waves
    attend_bf16<false, NW>(a, sel, pair, 0, a.n_chunks, wave, NW, wave, u.m);
    __syncthreads();
    merge_waves_and_store<KIN_BF16, NW>(a, u.m, pair, 0);
}

bool step_single_kernel(const Geo &g, int k, int num_cu) {
    const int cu = num_cu > 0 ? num_cu : 256;
    return g.dtype == KIN_BF16 && g.nb <= kStepMaxBlocks && k <= kStepIdxCap && g.pairs >= cu;
}

hipError_t launch_decode_step(const Geo &g, const void *q, const void *K, const void *V, void *S,
                              double *scores, int k, int32_t *idx, void *out, hipStream_t s) {
    AttnPlan p;
    const int keff = k < g.nb ? k : g.nb;
    p.n_tokens = keff * g.block;
    p.n_chunks = (p.n_tokens + kChunkBf16 - 1) / kChunkBf16;
    p.nsplit = 1;
    p.fused = 1;
    p.ws_bytes = 0;
    AttnArgs a;
    fill_args(a, g, p, q, K, V, nullptr, k, out, nullptr);
    StepExtra x{S, scores, idx, g.nb_cap};
    dim3 grid(g.pairs);
    switch (select_kpt(g.nb, kStepThreads)) {
    case 1: k_decode_step<1><<<grid, kStepThreads, 0, s>>>(a, x); break;
    case 2: k_decode_step<2><<<grid, kStepThreads, 0, s>>>(a, x); break;
    case 4: k_decode_step<4><<<grid, kStepThreads, 0, s>>>(a, x); break;
    case 8: k_decode_step<8><<<grid, kStepThreads, 0, s>>>(a, x); break;
    default: k_decode_step<16><<<grid, kStepThreads, 0, s>>>(a, x); break;
    }
    return hipGetLastError();
}

}  // namespace kin
