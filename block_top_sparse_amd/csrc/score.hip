// score.hip -- K2: block scores (and, in the decode-step form, the summary
// update of the newest block fused in front of them).
//
// The group score of block j for (sequence b, KV head g) is
//     sigma_j = sum_{h : h / gqa == g} q_h . s_j = (sum_h q_h) . s_j
// (the page's "mean score per block" of BlockTopKAttention, skill summary
// "Kinetics: Memory-Aware Test-Time Scaling", Implementation, summed over
// the query heads that share the KV head).  The scale 1/sqrt(d) is left out:
// it does not change the order.  Arithmetic is fp64, so rounding cannot
// reorder two blocks whose scores differ by more than ~1e-15 relative.
//
// This kernel streams every summary row once, which is the part of a
// sparse step that still grows with the context length, so it is written
// as a pure HBM stream:
//   - 16 lanes own one block row, 8 channels (16 B of bf16 / 32 B of fp32)
//     per lane, so one wave load covers 4 whole consecutive rows (1 KiB of
//     bf16); a wave issues all TPW x 4 loads of its rows before any math,
//     with the nontemporal hint (the rows are read once);
//   - each lane forms its 8-term fp64 partial in a fixed order, and the 16
//     partials of 4 blocks are folded with a reduce-scatter butterfly
//     (xor 8, 4, 2, 1).  The summation tree is the same for every block, so
//     two blocks with identical summaries get bit-identical scores and a tie
//     between them is decided by index alone.
//
// Decode-step form (UPDATE): workgroup x = 0 of each pair recomputes the
// summary of the newest block (ctx_len - 1 lies in it), writes it to S and
// scores it with the same per-lane math and the same butterfly; every other
// workgroup scores its range of blocks and leaves the newest block alone.
#include "attn_impl.h"
#include "scoring.h"

namespace kin {

// bf16: score tiles.  One 512-thread workgroup scores tile_rows consecutive
// blocks of one pair with the streaming loop of the decode step
// (scoring.h: 16-block batches, the 8 waves on consecutive batches, a ring
// of 4 batches in flight per wave); with UPDATE the tile holding the newest
// block rebuilds that block's summary first.  About one tile per CU, so a
// few pairs still spread over the whole chip.
constexpr int kTileThreads = 512;
// blocks of a score tile whose scores stay in LDS for the tile's own
// selection (tile candidates)
constexpr int kTileCandRows = 2048;

// Score tiles per pair and blocks per tile: about one workgroup per CU,
// rows a multiple of one round of the 8 waves.
static void tile_geometry(const Geo &g, int num_cu, int &tiles, int &rows) {
    constexpr int kRows = (kTileThreads / 64) * kScoreBatch;
    const int cu = num_cu > 0 ? num_cu : 256;
    tiles = g.pairs >= cu ? 1 : (cu + g.pairs - 1) / g.pairs;
    rows = (g.nb + tiles - 1) / tiles;
    rows = (rows + kRows - 1) / kRows * kRows;
    tiles = (g.nb + rows - 1) / rows;
}

TileCands step_tile_cands(const Geo &g, int k, int num_cu) {
    TileCands t{0, 0, 0};
    // every sequence of one length (a shorter one could keep all its blocks,
    // fewer than k), and the tiles' k best together fewer than the blocks.
    // Only for more than 8 blocks per thread of the selecting workgroup:
    // below that its selection is short, and the tiles' own selections cost
    // more than they save (measured: 2048 blocks per pair +1.7%, 4096 even,
    // 8192 -4 to -7%)
    if (g.dtype != KIN_BF16 || g.ctx_lens || k < 1 || k >= g.nb || k > kStepIdxCap ||
        g.nb <= 8 * kStepThreads)
        return t;
    int tiles, rows;
    tile_geometry(g, num_cu, tiles, rows);
    if (tiles < 2 || rows > kTileCandRows || (long long)tiles * k >= g.nb) return t;
    t.tiles = tiles;
    t.rows = rows;
    t.n = tiles * k;
    return t;
}

// CKPT > 0 (tile candidates): the tile's scores stay in LDS, counted into
// its own sign/exponent tables, and the tile selects its k best (ties to
// the lower block) with select.h, CKPT keys per thread.  A block among the
// pair's top k has fewer than k blocks of the pair ahead of it, so fewer
// than k of its tile: it is among its tile's k best.  The tile writes only
// those: their scores to `scores` and their block numbers to cand_idx
// ([pair][tile][k], ascending; past the tile's blocks -inf and -1).
template <bool UPDATE, bool SHARED, int CKPT>
__global__ __launch_bounds__(kTileThreads) void k_score_tiles(AttnArgs a0, void *S,
                                                             double *scores, int nb_cap,
                                                             int tile_rows, uint64_t *ctrl_zero,
                                                             int newest_only, int32_t *cand_idx) {
    constexpr int NW = kTileThreads / 64;
    static_assert(NewestLds<NW>::kMaxBlock >= 128, "every block size");
    static_assert(CKPT * kTileThreads <= kTileCandRows || CKPT == 0, "tile scores in LDS");
    __shared__ NewestLds<NW> nl;
    const int pair = blockIdx.y;
    // the pair's arrival word for the next kernel's in-kernel combine starts
    // at zero (kernels on one stream run in order)
    if (ctrl_zero && blockIdx.x == 0 && threadIdx.x == 0) ctrl_zero[pair] = 0ull;
    const AttnArgs a = for_pair(a0, pair);  // this sequence's own length
    const int nb = a.nb;
    if constexpr (CKPT > 0) {
        __shared__ double tsc[kTileCandRows];
        __shared__ SelectLds<CKPT, kTileThreads> sl;
        __shared__ int32_t tsel[kStepIdxCap];
        const int k = a.k;
        const int j_beg = blockIdx.x * tile_rows;  // every tile holds blocks
        const int j_end = min(nb, j_beg + tile_rows);
        select_clear(sl);
        if (threadIdx.x == 0) nl.ready = 0u;
        __syncthreads();
        auto emit = [&](int j, double v) {
            tsc[j - j_beg] = v;
            select_count(sl, v);
        };
        if (UPDATE && j_end == nb)
            score_blocks<NW, true, decltype(emit), false, SHARED>(a, S, nb_cap, pair, j_beg, nb,
                                                                  nl, emit);
        else
            score_blocks<NW, false, decltype(emit), false, SHARED>(a, S, nb_cap, pair, j_beg,
                                                                   j_end, nl, emit);
        __syncthreads();
        select_topk<CKPT, kTileThreads, true>(tsc, j_end - j_beg, k, tsel, sl);
        __syncthreads();
        const size_t c0 = ((size_t)pair * gridDim.x + blockIdx.x) * k;
        for (int i = threadIdx.x; i < k; i += kTileThreads) {
            const int l = tsel[i];
            scores[c0 + i] = l >= 0 ? tsc[l] : -__builtin_huge_val();
            cand_idx[c0 + i] = l >= 0 ? j_beg + l : -1;
        }
        return;
    }
    // newest_only: every block is kept and no scores are wanted, so only the
    // newest block's summary is rebuilt (by tile 0)
    const int j_beg = newest_only ? (blockIdx.x == 0 ? nb - 1 : nb) : blockIdx.x * tile_rows;
    if (j_beg >= nb) return;  // a shorter sequence: nothing left for this tile
    const int j_end = min(nb, j_beg + tile_rows);
    double *sp = scores + (size_t)pair * nb_cap;
    auto emit = [&](int j, double v) { sp[j] = v; };
    if (UPDATE && j_end == nb) {
        if (threadIdx.x == 0) nl.ready = 0u;
        __syncthreads();
        score_blocks<NW, true, decltype(emit), false, SHARED>(a, S, nb_cap, pair, j_beg, nb, nl,
                                                              emit);
    } else {
        score_blocks<NW, false, decltype(emit), false, SHARED>(a, S, nb_cap, pair, j_beg, j_end,
                                                               nl, emit);
    }
}

static hipError_t launch_tiles(const Geo &g, bool update, const void *q, const void *K, void *S,
                               double *scores, int num_cu, hipStream_t s, bool newest_only,
                               uint64_t *ctrl_zero, const TileCands *tc, int32_t *cand_idx,
                               int k) {
    AttnArgs a{};
    a.q = q;
    a.K = K;
    a.hkv = g.hkv;
    a.gqa = g.gqa;
    a.t_cap = g.t_cap;
    a.ctx_len = g.ctx_len;
    a.block = g.block;
    a.block_shift = __builtin_ctz((unsigned)g.block);
    a.nb = g.nb;
    a.k = tc ? k : 1;  // the tiles' own selection (else unused)
    a.ctx_lens = g.ctx_lens;
    a.Sp = g.Sp;
    a.share_n = g.share_n;
    a.prompt_len = g.prompt_len;
    a.prompt_blocks = g.share_n ? g.prompt_len / g.block : 0;
    a.pages = g.pages;
    a.page_shift = g.page_shift;
    a.max_pages = g.max_pages;
    a.num_pages = g.num_pages;
    int tiles, rows;
    tile_geometry(g, num_cu, tiles, rows);
    const dim3 grid(newest_only ? 1 : tiles, g.pairs);
    const int no = newest_only ? 1 : 0;
    if (tc) {  // tile candidates: the first kernel of the decode step
#define KIN_TILES_CAND(SH, C)                                                                  \
    k_score_tiles<true, SH, C><<<grid, kTileThreads, 0, s>>>(a, S, scores, g.nb_cap, rows,     \
                                                             ctrl_zero, 0, cand_idx)
#define KIN_TILES_CAND_KPT(SH)                                                                 \
    do {                                                                                       \
        switch (select_kpt(rows, kTileThreads)) {                                              \
        case 1: KIN_TILES_CAND(SH, 1); break;                                                  \
        case 2: KIN_TILES_CAND(SH, 2); break;                                                  \
        default: KIN_TILES_CAND(SH, 4); break;                                                 \
        }                                                                                      \
    } while (0)
        if (g.share_n)
            KIN_TILES_CAND_KPT(true);
        else
            KIN_TILES_CAND_KPT(false);
#undef KIN_TILES_CAND_KPT
#undef KIN_TILES_CAND
    } else if (update && g.share_n) {
        k_score_tiles<true, true, 0><<<grid, kTileThreads, 0, s>>>(a, S, scores, g.nb_cap, rows,
                                                                   ctrl_zero, no, nullptr);
    } else if (update) {
        k_score_tiles<true, false, 0><<<grid, kTileThreads, 0, s>>>(a, S, scores, g.nb_cap, rows,
                                                                    ctrl_zero, no, nullptr);
    } else {
        k_score_tiles<false, false, 0><<<grid, kTileThreads, 0, s>>>(a, S, scores, g.nb_cap,
                                                                     rows, ctrl_zero, 0, nullptr);
    }
    return hipGetLastError();
}

template <int DT, int TPW, bool UPDATE>
__global__ __launch_bounds__(256) void k_block_score(const void *__restrict__ qv,
                                                     const void *__restrict__ Kv, void *Sv,
                                                     double *__restrict__ scores, int hkv,
                                                     int gqa, int t_cap, int nb_cap, int nb,
                                                     int ctx_len, int block,
                                                     uint64_t *ctrl_zero) {
    constexpr int kBlocksPerWave = 16 * TPW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane & 15;  // channel slice: channels 8*sub .. 8*sub+7
    const int grp = lane >> 4;  // which of the 4 rows of a wave load
    const int pair = blockIdx.y;
    const int b = pair / hkv, g = pair % hkv;
    const size_t row0 = (size_t)pair * nb_cap;
    const int newest = nb - 1;
    // the pair's arrival word for the next kernel's in-kernel combine starts
    // at zero (kernels on one stream run in order)
    if (ctrl_zero && blockIdx.x == 0 && threadIdx.x == 0) ctrl_zero[pair] = 0ull;

    if (UPDATE && blockIdx.x == 0) {
        __shared__ uint32_t row_lds[kHeadDim];
        if (wave == 0)
            newest_summary<DT>(Kv, Sv, pair, t_cap, nb_cap, ctx_len, block, row_lds, lane);
        __syncthreads();
        if (wave != 0) return;
        double qs[8];
        group_query_sum<DT>(qv, b, g, hkv, gqa, sub, qs);
        // the newest row sits in slot u = 0 of row group 0; the other slots
        // are zero rows, so the butterfly is the one every block goes through
        u32x4 a = {0u, 0u, 0u, 0u}, c = {0u, 0u, 0u, 0u};
        if (grp == 0) {
            const uint32_t *r = row_lds + (DT == KIN_BF16 ? 4 : 8) * sub;
            a = u32x4{r[0], r[1], r[2], r[3]};
            if (DT != KIN_BF16) c = u32x4{r[4], r[5], r[6], r[7]};
        }
        double part[4];
        part[0] = slice_dot<DT>(qs, a, c);
        part[1] = part[2] = part[3] = slice_dot<DT>(qs, u32x4{0u, 0u, 0u, 0u},
                                                    u32x4{0u, 0u, 0u, 0u});
        const double x = fold4(part, lane);
        if (lane == 0) store_score(scores, row0 + newest, x);
        return;
    }

    // With UPDATE the newest row is rewritten by workgroup 0 during this
    // launch, so no other workgroup loads it (a store to it while loads of
    // the same lines are in flight can be lost): they cover rows < nb - 1.
    const int n_rows = UPDATE ? nb - 1 : nb;
    const int wave_j0 = ((blockIdx.x - (UPDATE ? 1 : 0)) * 4 + wave) * kBlocksPerWave;
    if (wave_j0 >= n_rows) return;
    double qs[8];
    group_query_sum<DT>(qv, b, g, hkv, gqa, sub, qs);

    // every row load of the wave is issued before any arithmetic
    u32x4 wa[TPW][4], wb[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = min(wave_j0 + 16 * t + 4 * u + grp, n_rows - 1);
            load_row_slice<DT>(Sv, row0 + j, sub, wa[t][u], wb[t][u]);
        }
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        double part[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) part[u] = slice_dot<DT>(qs, wa[t][u], wb[t][u]);
        const double x = fold4(part, lane);
        const int u = ((lane & 8) ? 2 : 0) + ((lane & 4) ? 1 : 0);
        const int j = wave_j0 + 16 * t + 4 * u + grp;
        if ((lane & 3) == 0 && j < n_rows) store_score(scores, row0 + j, x);
    }
}

template <int DT, bool UPDATE>
static hipError_t launch_dt(const Geo &g, const void *q, const void *K, void *S, double *scores,
                            hipStream_t s, uint64_t *ctrl_zero) {
    // blocks per workgroup = 4 waves x 16 x TPW; smaller workgroups when the
    // problem is small so the grid still covers the chip
    const long long total = (long long)g.pairs * g.nb;
    const int extra = UPDATE ? 1 : 0;
#define KIN_SCORE_LAUNCH(TPW)                                                                    \
    k_block_score<DT, TPW, UPDATE><<<dim3((g.nb + 64 * TPW - 1) / (64 * TPW) + extra, g.pairs), \
                                     256, 0, s>>>(q, K, S, scores, g.hkv, g.gqa, g.t_cap,         \
                                                  g.nb_cap, g.nb, g.ctx_len, g.block, ctrl_zero)
    if (total >= 2048LL * 256)
        KIN_SCORE_LAUNCH(4);
    else if (total >= 2048LL * 128)
        KIN_SCORE_LAUNCH(2);
    else
        KIN_SCORE_LAUNCH(1);
#undef KIN_SCORE_LAUNCH
    return hipGetLastError();
}

hipError_t launch_block_score(const Geo &g, const void *q, const void *S, double *scores,
                              int num_cu, hipStream_t s) {
    void *Sm = const_cast<void *>(S);  // not written without UPDATE
    return g.dtype == KIN_BF16
               ? launch_tiles(g, false, q, nullptr, Sm, scores, num_cu, s, false, nullptr,
                              nullptr, nullptr, 0)
               : launch_dt<KIN_F32, false>(g, q, nullptr, Sm, scores, s, nullptr);
}

hipError_t launch_update_and_score(const Geo &g, const void *q, const void *K, void *S,
                                   double *scores, int num_cu, hipStream_t s, bool newest_only,
                                   uint64_t *ctrl_zero, const TileCands *tc, int32_t *cand_idx,
                                   int k) {
    return g.dtype == KIN_BF16 ? launch_tiles(g, true, q, K, S, scores, num_cu, s, newest_only,
                                              ctrl_zero, tc, cand_idx, k)
                               : launch_dt<KIN_F32, true>(g, q, K, S, scores, s, ctrl_zero);
}

}  // namespace kin
