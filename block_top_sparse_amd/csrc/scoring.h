// scoring.h -- the scoring phase of a decode step, run by one workgroup of
// NW waves over a range of a pair's blocks: the fp64 group scores of the
// blocks (skill summary "Kinetics: Memory-Aware Test-Time Scaling",
// Implementation: the mean-score-per-block of BlockTopKAttention, here
// (sum of the group's queries) . (mean key of the block)), and, when the
// range holds the newest block, that block's summary rebuilt from K first.
//
// Memory pattern: the summary rows stream in 16-block batches (16 lanes per
// row, 4 rows per 1 KiB load); the NW waves of the workgroup read
// consecutive batches, so one round covers 16 * NW consecutive rows, and
// each wave keeps kRing batches in flight (a ring: a batch's slot is
// refilled right after its math).  Every load is unconditional (rows past
// the range re-read a row that is never written during the step, and are
// never used), so the compiler's wait before each batch's math covers
// exactly that batch's loads.
//
// Shared by the single-kernel decode step (step.hip) and the score tiles of
// the scoring calls (score.hip).
#pragma once

#include "attn_impl.h"
#include "score_impl.h"

namespace kin {

constexpr int kQPre = 8;    // query rows of the group requested up front
constexpr int kRing = 4;    // summary batches in flight per wave
constexpr int kKPre = 16;   // newest-block K rows each wave stages
constexpr int kScoreBatch = 16;  // blocks per wave per batch

// LDS of the newest-block rebuild: the block's K rows (each wave stages
// kKPre of them), the count of threads that have staged theirs, the new row.
// Holds blocks of up to kMaxBlock tokens (8 waves: every block size; the
// launchers choose fewer waves only for blocks that fit).
template <int NW>
struct NewestLds {
    static constexpr int kMaxBlock = NW * kKPre;
    uint32_t k[NW * kKPre][kHeadDim / 2];
    uint32_t row[kHeadDim / 2];
    uint32_t row2[kHeadDim / 2];  // Quest summaries: the maximum row
    uint32_t ready;
};

// Load the 16-block batch starting at j0: 16 lanes per row, 4 rows per
// load (one 1 KiB request), 4 loads.  Row j is at rows + j rows; with SPLIT,
// rows below j_split (a shared prompt's summaries) are at rows_lo + j rows.
// Rows past j_max re-read row j_max.
template <bool SPLIT>
__device__ __forceinline__ void load_batch(const uint16_t *rows_lo, const uint16_t *rows,
                                           int j_split, int j0, int j_max, int sub, int grp,
                                           u32x4 (&w)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = min(j0 + 4 * u + grp, j_max);
        const uint16_t *base = (SPLIT && j < j_split) ? rows_lo : rows;
        w[u] = ld_nt16(base + (size_t)j * kHeadDim + 8 * sub);
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

// The Quest form: only the positive parts of the slice (pos) or only the
// negative parts.  A head's bound max(q*min, q*max) summed over the group's
// heads is P . max + N . min, P and N the sums of the heads' positive and
// negative query parts.
__device__ __forceinline__ void add_q_slice_signed(double (&qs)[8], const u32x4 &w, bool on,
                                                   bool pos) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double lo = (double)bf16_lo(w[e]), hi = (double)bf16_hi(w[e]);
        qs[2 * e] += on ? (pos ? fmax(lo, 0.0) : fmin(lo, 0.0)) : 0.0;
        qs[2 * e + 1] += on ? (pos ? fmax(hi, 0.0) : fmin(hi, 0.0)) : 0.0;
    }
}

// Scores of one batch (blocks j0 .. j0+15): lane 4m holds the score of
// block j0 + batch_offset(4m) (the other lanes hold partial sums).
__device__ __forceinline__ double score_batch(const double (&qs)[8], const u32x4 (&w)[4],
                                              int lane) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    double part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) part[u] = slice_dot<KIN_BF16>(qs, w[u], zero);
    return fold4(part, lane);
}

// Offset inside its batch of the block whose score lane 4m holds.
__device__ __forceinline__ int batch_offset(int lead) {
    const int u = ((lead & 8) ? 2 : 0) + ((lead & 4) ? 1 : 0);
    return 4 * u + (lead >> 4);
}

// Lane 4m + r takes the value lane 4m holds in x[r] (a DPP broadcast inside
// each quad per slot, then a select): kRing batch scores spread over all 64
// lanes, so one round of the ring is handed out with one emit per lane.
static_assert(kRing == 4, "one ring round: one slot per lane of a quad");
__device__ __forceinline__ double quad_gather(const double (&x)[kRing], int r) {
    double out = 0.0;
#pragma unroll
    for (int s = 0; s < kRing; ++s) {
        const uint64_t b = (uint64_t)__double_as_longlong(x[s]);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, 0x00, 0xF,
                                                                  0xF, false);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), 0x00,
                                                                  0xF, 0xF, false);
        const double v = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
        out = r == s ? v : out;
    }
    return out;
}

// Blocks [j_beg, j_end) of pair `pair` (bf16 cache; `a` already holds the
// pair's own length, for_pair).  NEWEST: the range ends
// with the newest block nb - 1 (ctx_len - 1 lies in it): its summary is
// rebuilt (fp64 sum in ascending token order, fp64 mean, fp32 then bf16
// rounding), written to S and scored by wave 0 after its batches, with the
// same math as every other block.  Requires, when NEWEST, nl.ready == 0 and
// a barrier since.  Ends without a barrier.
//
// QUEST: the summaries are [pair][nb_cap][2][d] (channel-wise minimum row,
// then maximum row) and a block's score is the Quest bound P . max + N .
// min: the loop runs over rows, lanes of even row groups hold N (minimum
// rows land there), odd ones P, and the two rows of a block are added
// after the fold.  The newest block's rows are its keys' minimum and
// maximum (ascending token order, the first of equal values kept).
// SHARED: the sequences share prompts (AttnArgs::share_n), whose blocks'
// summaries come from the prompt's own array.
template <int NW, bool NEWEST, class Emit, bool QUEST = false, bool SHARED = false>
__device__ void score_blocks(const AttnArgs &a, void *Sv, int nb_cap, int pair, int j_beg,
                             int j_end, NewestLds<NW> &nl, Emit emit) {
    constexpr int RB = QUEST ? 2 : 1;  // summary rows per block
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane & 15, grp = lane >> 4;
    const int b = pair / a.hkv, g = pair % a.hkv;
    const int nb = a.nb;
    const size_t row0 = (size_t)pair * nb_cap * RB;
    const uint16_t *S = static_cast<const uint16_t *>(Sv);
    const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                         ((size_t)b * a.hkv * a.gqa + (size_t)g * a.gqa) * kHeadDim + 8 * sub;
    constexpr int kStride = NW * kScoreBatch;
    // (rows: RB per block; the newest block is scored apart)
    const int j_lim = RB * (NEWEST ? nb - 1 : j_end);
    const int jw = RB * j_beg + wave * kScoreBatch;
    const int n = jw < j_lim ? (j_lim - jw + kStride - 1) / kStride : 0;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // Rows loaded past the range (the ring's spare loads) re-read a row that
    // nothing writes during the step: the last scored row, else the row
    // before the range, else (a range holding only the newest block of a
    // one-block context) row 0 of the pair's K.  Never the newest block's
    // row: a store to it while loads of the same lines are in flight can be
    // lost.
    const int j_safe = j_lim > RB * j_beg ? j_lim - 1 : RB * j_beg - 1;
    const uint16_t *rows = j_safe >= 0 ? S + row0 * kHeadDim
                                       : static_cast<const uint16_t *>(a.K) +
                                             token_row(a, pair, 0) * kHeadDim;
    const int j_max = j_safe >= 0 ? j_safe : 0;
    // a shared prompt's blocks come from its own summary array
    static_assert(!(QUEST && SHARED), "shared prompts use mean-key summaries");
    const int j_split = SHARED ? a.prompt_blocks : 0;
    const uint16_t *rows_lo =
        SHARED ? static_cast<const uint16_t *>(a.Sp) +
                        (size_t)prompt_unit(a, pair) * a.prompt_blocks * kHeadDim
                  : rows;

    // Issue order: query rows, this wave's share of the newest block's K
    // rows, batches 0 .. kRing - 1.
    u32x4 qw[kQPre];
#pragma unroll
    for (int r = 0; r < kQPre; ++r)
        qw[r] = *reinterpret_cast<const u32x4 *>(qp + min(r, a.gqa - 1) * kHeadDim);
    const int jn = nb - 1;
    const int tn = min(a.block, a.ctx_len - jn * a.block);
    const int tw = wave * kKPre;
    uint32_t kw[kKPre];
    if (NEWEST) {
        // the block lies inside one page: its rows are consecutive
        const uint32_t *kn = static_cast<const uint32_t *>(a.K) +
                             token_row(a, pair, jn * a.block) * (kHeadDim / 2) + lane;
#pragma unroll
        for (int t = 0; t < kKPre; ++t) kw[t] = kn[(size_t)min(tw + t, tn - 1) * (kHeadDim / 2)];
    }
    u32x4 w[kRing][4];
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
        load_batch<SHARED>(rows_lo, rows, j_split, jw + r * kStride, j_max, sub, grp, w[r]);
        // keep slot order: the loop's waits assume slot 0 was issued first
        __builtin_amdgcn_sched_barrier(0);
    }

    // group query sum, heads in ascending order (fp64)
    double qs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[e] = 0.0;
    if constexpr (QUEST) {
        const bool pos = (grp & 1) != 0;  // odd row groups hold maximum rows
#pragma unroll
        for (int r = 0; r < kQPre; ++r) add_q_slice_signed(qs, qw[r], r < a.gqa, pos);
        for (int r = kQPre; r < a.gqa; ++r)
            add_q_slice_signed(qs, *reinterpret_cast<const u32x4 *>(qp + r * kHeadDim), true, pos);
    } else {
#pragma unroll
        for (int r = 0; r < kQPre; ++r) add_q_slice(qs, qw[r], r < a.gqa);
        for (int r = kQPre; r < a.gqa; ++r)
            add_q_slice(qs, *reinterpret_cast<const u32x4 *>(qp + r * kHeadDim), true);
    }

    if (NEWEST) {
        // stage this wave's K rows (rows past the block are never read);
        // every thread releases its own stores with its own increment
#pragma unroll
        for (int t = 0; t < kKPre; ++t) nl.k[tw + t][lane] = kw[t];
        __hip_atomic_fetch_add(&nl.ready, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    // batch i is scored from slot i % kRing, which then takes batch i + kRing;
    // every round scores all kRing slots (a batch past the range emits
    // nothing) and refills them unconditionally
    for (int i0 = 0; i0 < n; i0 += kRing) {
        double x[kRing];
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            x[r] = score_batch(qs, w[r], lane);
            if constexpr (QUEST) x[r] += __shfl_xor(x[r], 16);  // minimum row + maximum row
            load_batch<SHARED>(rows_lo, rows, j_split, jw + (i0 + r + kRing) * kStride, j_max,
                               sub, grp, w[r]);
        }
        // lane 4m + r: the score of block batch_offset(4m) of slot r's batch
        // (one emit per lane and round; -0.0 becomes +0.0)
        {
            const int r = lane & 3;
            double v = quad_gather(x, r);
            const int j = jw + (i0 + r) * kStride + batch_offset(lane & ~3);
            if (j < j_lim && (!QUEST || (grp & 1) == 0)) {
                if (v == 0.0) v = 0.0;
                emit(j / RB, v);
            }
        }
    }
    // The last refills are used after the loop as well (an empty asm reads
    // them), so the compiler cannot sink them below the loop test, where
    // they would become conditional and every wait would turn strict.
#pragma unroll
    for (int r = 0; r < kRing; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v)
            asm volatile("" ::"v"(w[r][v][0]), "v"(w[r][v][1]), "v"(w[r][v][2]), "v"(w[r][v][3]));

    if (NEWEST && wave == 0) {
        // wait for all NW * 64 threads' stores (every wave stages its rows
        // before its first batch, so this wait is normally already over)
        while (__hip_atomic_load(&nl.ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <
               (uint32_t)(NW * 64))
            __builtin_amdgcn_s_sleep(1);
        if constexpr (QUEST) {
            // channel-wise minimum and maximum (16-bit halves: channels 2 lane,
            // 2 lane + 1), strict comparisons in token order
            uint32_t v0 = nl.k[0][lane];
            float lo0 = bf16_lo(v0), hi0 = lo0, lo1 = bf16_hi(v0), hi1 = lo1;
            uint32_t blo0 = v0 & 0xFFFFu, bhi0 = blo0, blo1 = v0 >> 16, bhi1 = blo1;
            for (int t = 1; t < tn; ++t) {
                const uint32_t v = nl.k[t][lane];
                const float x0 = bf16_lo(v), x1 = bf16_hi(v);
                if (x0 < lo0) { lo0 = x0; blo0 = v & 0xFFFFu; }
                if (x0 > hi0) { hi0 = x0; bhi0 = v & 0xFFFFu; }
                if (x1 < lo1) { lo1 = x1; blo1 = v >> 16; }
                if (x1 > hi1) { hi1 = x1; bhi1 = v >> 16; }
            }
            const uint32_t vmin = blo0 | (blo1 << 16), vmax = bhi0 | (bhi1 << 16);
            static_cast<uint32_t *>(Sv)[(row0 + 2 * (size_t)jn) * (kHeadDim / 2) + lane] = vmin;
            static_cast<uint32_t *>(Sv)[(row0 + 2 * (size_t)jn + 1) * (kHeadDim / 2) + lane] = vmax;
            nl.row[lane] = vmin;
            nl.row2[lane] = vmax;
        } else {
            double s0 = 0.0, s1 = 0.0;  // lane = channels 2 lane, 2 lane + 1
#pragma unroll 16
            for (int t = 0; t < tn; ++t) {
                const uint32_t v = nl.k[t][lane];
                s0 += (double)bf16_lo(v);
                s1 += (double)bf16_hi(v);
            }
            const double cnt = (double)tn;
            const float m0 = (float)(s0 / cnt), m1 = (float)(s1 / cnt);
            const uint32_t v = f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
            static_cast<uint32_t *>(Sv)[(row0 + jn) * (kHeadDim / 2) + lane] = v;
            nl.row[lane] = v;
        }

        // the newest row in slot u = 0 of row group 0 (Quest: its minimum row
        // there, its maximum row in row group 1), zero rows elsewhere: the
        // butterfly every block goes through
        u32x4 r = zero;
        if (grp == 0 || (QUEST && grp == 1)) {
            const uint32_t *p = (QUEST && grp == 1 ? nl.row2 : nl.row) + 4 * sub;
            r = u32x4{p[0], p[1], p[2], p[3]};
        }
        double part[4];
        part[0] = slice_dot<KIN_BF16>(qs, r, zero);
        part[1] = part[2] = part[3] = slice_dot<KIN_BF16>(qs, zero, zero);
        double x = fold4(part, lane);
        if constexpr (QUEST) x += __shfl_xor(x, 16);
        if (lane == 0) {
            if (x == 0.0) x = 0.0;
            emit(jn, x);
        }
    }
}

}  // namespace kin
