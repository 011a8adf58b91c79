// step.hip -- a whole block top-k sparse decode step in ONE kernel, one
// 512-thread workgroup per (sequence, KV head) pair:
//
//   1. wave 0 rebuilds the summary of the newest block (fp64 mean in token
//      order, rounded to bf16) and writes it to S, while
//   2. all 8 waves score every other block of the pair against the group's
//      query sum (fp64, the same per-lane math and butterfly as the
//      standalone scoring kernel); wave 0 then scores the newest block from
//      its new row; the scores stay in LDS (and are written out);
//   3. the workgroup selects the top k blocks from LDS (select.h; the
//      exponent count tables are filled while the scores are made);
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
constexpr int kQPre = 8;   // query rows of the group requested up front
constexpr int kRing = 4;   // summary batches in flight per wave while scoring
constexpr int kKPre = 16;  // newest-block K rows each wave stages (8 x 16 >= 128 tokens)

struct StepExtra {
    void *S;
    double *scores;  // may be null: the scores are then not written out
    int32_t *idx;
    int nb_cap;
};

// Load this wave's 16-block batch starting at j0: 16 lanes per row, 4 rows
// per load (one 1 KiB request), 4 loads.  Rows past nb re-read row nb - 1
// (never used).
__device__ __forceinline__ void load_batch(const uint16_t *S, size_t row0, int j0, int nb,
                                           int sub, int grp, u32x4 (&w)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = min(j0 + 4 * u + grp, nb - 1);
        w[u] = ld_nt16(S + (row0 + j) * kHeadDim + 8 * sub);
    }
}

// qs[0..8) += the 8 channels of one bf16 query slice if `on`, else += 0.0
// (exact: the sums start at +0.0, so they are never -0.0).  A select, not a
// branch, so the slice's load is not moved next to its use.
__device__ __forceinline__ void add_q_slice(double (&qs)[8], const u32x4 &w, bool on) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        qs[2 * e] += on ? (double)bf16_lo(w[e]) : 0.0;
        qs[2 * e + 1] += on ? (double)bf16_hi(w[e]) : 0.0;
    }
}

template <class Sel>
__device__ __forceinline__ void score_batch(const double (&qs)[8], const u32x4 (&w)[4], int j0,
                                            int nb, int lane, int grp, double *sc_lds,
                                            double *sc_out, Sel &sl) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    double part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) part[u] = slice_dot<KIN_BF16>(qs, w[u], zero);
    double x = fold4(part, lane);
    const int u = ((lane & 8) ? 2 : 0) + ((lane & 4) ? 1 : 0);
    const int j = j0 + 4 * u + grp;
    if ((lane & 3) == 0 && j < nb - 1) {  // the newest block is scored apart
        if (x == 0.0) x = 0.0;  // one zero: -0.0 becomes +0.0
        sc_lds[j] = x;
        if (sc_out) sc_out[j] = x;  // scores are an optional output
        select_count(sl, x);
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

    // the newest block's K rows, staged in LDS by all waves (16 rows each);
    // wave 0 sums them in token order once every wave has stored its share
    static_assert(kStepThreads / 64 * kKPre >= 128, "the largest block must fit");
    __shared__ uint32_t newest_k[kStepThreads / 64 * kKPre][kHeadDim / 2];
    __shared__ uint32_t newest_ready;
    __shared__ uint32_t newest_row[kHeadDim / 2];
    select_clear(sl);
    if (tid == 0) newest_ready = 0u;
    __syncthreads();

    // 1+2. every wave scores its 64-block batches of the pair; wave 0 also
    // rebuilds the newest block's summary and scores that block last from
    // the LDS copy of the new row (same math); the batches skip it.
    {
        const int sub = lane & 15, grp = lane >> 4;
        const uint16_t *S = static_cast<const uint16_t *>(x.S);
        const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                             ((size_t)b * a.hkv * a.gqa + (size_t)g * a.gqa) * kHeadDim + 8 * sub;
        double *sc_out = x.scores ? x.scores + row0 : nullptr;
        constexpr int kBatch = 16;  // blocks per wave per batch
        constexpr int kStride = NW * kBatch;  // the 8 waves read 128 consecutive rows
        const int jw = wave * kBatch;
        const int n = jw < nb ? (nb - jw + kStride - 1) / kStride : 0;
        const u32x4 zero = {0u, 0u, 0u, 0u};

        // Issue order: query rows, this wave's share of the newest block's
        // K rows, batches 0 .. kRing - 1.  The loads are unconditional (rows out
        // of range re-read the last valid one and are never used), so the
        // wait before each use covers exactly the loads issued before it.
        u32x4 qw[kQPre];
#pragma unroll
        for (int r = 0; r < kQPre; ++r)
            qw[r] = *reinterpret_cast<const u32x4 *>(qp + min(r, a.gqa - 1) * kHeadDim);
        const int jn = nb - 1;  // the newest block: ctx_len - 1 lies in it
        const int tn = min(a.block, a.ctx_len - jn * a.block);
        const int tw = wave * kKPre;
        const uint32_t *kn = static_cast<const uint32_t *>(a.K) +
                             ((size_t)pair * a.t_cap + (size_t)jn * a.block) * (kHeadDim / 2) + lane;
        uint32_t kw[kKPre];
#pragma unroll
        for (int t = 0; t < kKPre; ++t) kw[t] = kn[(size_t)min(tw + t, tn - 1) * (kHeadDim / 2)];
        u32x4 w[kRing][4];
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            load_batch(S, row0, jw + r * kStride, nb, sub, grp, w[r]);
            // keep slot order: the loop's waits assume slot 0 was issued first
            __builtin_amdgcn_sched_barrier(0);
        }

        // group query sum, heads in ascending order (fp64)
        double qs[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[e] = 0.0;
#pragma unroll
        for (int r = 0; r < kQPre; ++r) add_q_slice(qs, qw[r], r < a.gqa);
        for (int r = kQPre; r < a.gqa; ++r)
            add_q_slice(qs, *reinterpret_cast<const u32x4 *>(qp + r * kHeadDim), true);

        // stage this wave's K rows (rows past the block are never read)
#pragma unroll
        for (int t = 0; t < kKPre; ++t) newest_k[tw + t][lane] = kw[t];
        __hip_atomic_fetch_add(&newest_ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);

        // A ring of kRing batches: batch i is scored from slot i % kRing,
        // which then takes batch i + kRing.  Every round scores all kRing
        // slots and refills them unconditionally (a batch past the end
        // re-reads row nb - 1, an L2 hit, and stores no score), so the wait
        // before a batch's math covers only that batch's loads.
        for (int i0 = 0; i0 < n; i0 += kRing) {
#pragma unroll
            for (int r = 0; r < kRing; ++r) {
                score_batch(qs, w[r], jw + (i0 + r) * kStride, nb, lane, grp, u.sc, sc_out, sl);
                load_batch(S, row0, jw + (i0 + r + kRing) * kStride, nb, sub, grp, w[r]);
            }
        }
        // The last refills are used after the loop as well (an empty asm
        // reads them), so the compiler cannot sink them below the loop test,
        // where they would become conditional and every wait would turn
        // strict.
#pragma unroll
        for (int r = 0; r < kRing; ++r)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                asm volatile("" ::"v"(w[r][v][0]), "v"(w[r][v][1]), "v"(w[r][v][2]),
                             "v"(w[r][v][3]));
        if (wave == 0) {
            // newest summary: fp64 sum in ascending token order, fp64 mean,
            // then fp32 and bf16 rounding; lane = channels 2 lane, 2 lane + 1.
            // Every wave stores its rows before its first batch, so this wait
            // is normally already satisfied.
            while (__hip_atomic_load(&newest_ready, __ATOMIC_ACQUIRE,
                                     __HIP_MEMORY_SCOPE_WORKGROUP) < (uint32_t)NW)
                __builtin_amdgcn_s_sleep(1);
            double s0 = 0.0, s1 = 0.0;
#pragma unroll 16
            for (int t = 0; t < tn; ++t) {
                const uint32_t w = newest_k[t][lane];
                s0 += (double)bf16_lo(w);
                s1 += (double)bf16_hi(w);
            }
            const double cnt = (double)tn;
            const float m0 = (float)(s0 / cnt), m1 = (float)(s1 / cnt);
            const uint32_t w = f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
            static_cast<uint32_t *>(x.S)[(row0 + jn) * (kHeadDim / 2) + lane] = w;
            newest_row[lane] = w;

            // the newest row in slot u = 0 of row group 0, zero rows elsewhere
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
                if (sc_out) sc_out[nb - 1] = v;
                select_count(sl, v);
            }
        }
    }
    __syncthreads();

    // 3. selection (reads the scores from LDS; they are dead afterwards, so
    //    the merge area may reuse them)
    select_topk<KPT, kStepThreads, true>(u.sc, nb, a.k, sel, sl);
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
