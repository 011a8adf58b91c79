// kin_internal.h -- shared between the ABI layer and the kernel files of
// libkin.so.  Not installed; the public interface is include/kin.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kin.h"

namespace kin {

constexpr int kHeadDim = 128;  // the only head_dim built
constexpr int kMaxGqa = 16;    // query heads of one group fit one 16-row MFMA tile
constexpr int kMaxBlocks = 16384;
constexpr int kChunkBf16 = 32;  // tokens per wave iteration, bf16 attention
constexpr int kChunkF32 = 16;   // tokens per wave iteration, fp32 attention
constexpr int kStepIdxCap = 2048;  // kept blocks the select+attend kernels hold in LDS
constexpr int kTokIdxCap = 8192;   // kept tokens of the token-level step (LDS)
constexpr int kTokMaxLen = 262144;  // tokens of one pair the two-kernel token step takes

// Every workspace starts with kCtrlWords 64-bit arrival words (one per pair
// of a split launch, which runs only with fewer pairs than compute units):
// the caller zeroes a workspace once, and every call leaves these words at
// zero when it completes.  The rest of the workspace (partials, handed-over
// scores) follows them.
constexpr int kCtrlWords = 1024;
constexpr size_t kCtrlBytes = (size_t)kCtrlWords * sizeof(uint64_t);
// bytes of a workspace whose part after the arrival words is `body` bytes
inline size_t ws_total(size_t body) { return body ? kCtrlBytes + body : 0; }
// the part of a workspace after its arrival words
inline char *ws_body(void *ws) { return ws ? static_cast<char *>(ws) + kCtrlBytes : nullptr; }

// Geometry shared by the launchers (all derived from a validated desc).
struct Geo {
    int batch, hkv, gqa, hq, t_cap, ctx_len, block, dtype;
    int nb, nb_cap, pairs;
    // variable lengths / paged caches (null: every sequence holds ctx_len
    // tokens in a contiguous cache); ctx_len and nb are then upper bounds
    const int32_t *ctx_lens = nullptr;
    const int32_t *pages = nullptr;
    int page_shift = 0, max_pages = 0, num_pages = 0;
    // shared prompts (share_n == 0: none; see AttnArgs)
    const void *Kp = nullptr, *Vp = nullptr, *Sp = nullptr;
    int share_n = 0, prompt_len = 0;
};

// Split-KV plan of one attention call.
struct AttnPlan {
    int n_tokens;  // length of each pair's token list (kept blocks x block, or ctx_len)
    int n_chunks;  // ceil(n_tokens / chunk)
    int nsplit;    // workgroups per (sequence, KV head)
    int fused;     // decode step: selection and attention in one kernel
    size_t ws_bytes;
};

AttnPlan plan_attention(const Geo &g, int k, bool dense, int num_cu);

hipError_t launch_block_summary(const Geo &g, const void *K, void *S, int j0, int j1,
                                hipStream_t s);
// the same for variable lengths / paged caches (bf16): blocks of [t_begin,
// t_end) inside each sequence
hipError_t launch_block_summary_paged(const Geo &g, const void *K, void *S, int t_begin,
                                      int t_end, hipStream_t s);
hipError_t launch_block_score(const Geo &g, const void *q, const void *S, double *scores,
                              int num_cu, hipStream_t s);
// Tile candidates of the few-pair two-kernel step (bf16, one length for
// every sequence): when the score tiles of a pair fit in LDS and their k
// best together are fewer than the pair's blocks, each tile keeps its own
// k best (a superset of the pair's top k) and hands over only those.
// tiles == 0: not used; n = tiles * k candidates per pair.
struct TileCands {
    int tiles, rows, n;
};
TileCands step_tile_cands(const Geo &g, int k, int num_cu);
// decode step, first half: newest-block summary update + all block scores
// (bf16: newest_only skips the scores, for a step that keeps every block;
// ctrl_zero: arrival words, one per pair, to clear for the second half;
// tc: tile candidates instead of all scores, their scores to `scores` and
// their block numbers to cand_idx, [pair][tc->n] each)
hipError_t launch_update_and_score(const Geo &g, const void *q, const void *K, void *S,
                                   double *scores, int num_cu, hipStream_t s,
                                   bool newest_only = false, uint64_t *ctrl_zero = nullptr,
                                   const TileCands *tc = nullptr, int32_t *cand_idx = nullptr,
                                   int k = 0);
hipError_t launch_block_topk(const Geo &g, const double *scores, int k, int32_t *idx,
                             hipStream_t s);
hipError_t launch_attention(const Geo &g, const AttnPlan &p, const void *q, const void *K,
                            const void *V, const int32_t *idx, int k, void *out, void *ws,
                            hipStream_t s);
// decode step, second half: top-k selection + sparse attention, fused per
// pair when the plan allows it (plan_step); otherwise separate launches
AttnPlan plan_step(const Geo &g, int k, int num_cu);
// (the splits of a pair count their arrivals in the pair's word at
// step_ctrl(), which is zero on entry: cleared by an earlier kernel of the
// step or left at zero by the previous call; S_newest: with a fused plan
// that keeps every block, bf16, the summaries whose newest row the kernel
// rebuilds, so that no first half is needed)
// cand: the tile candidates' block numbers ([pair][n_cand]; scores then
// holds their scores in the same layout), or nullptr: scores holds every
// block's score ([pair][nb_cap])
hipError_t launch_select_attend(const Geo &g, const AttnPlan &p, const void *q, const void *K,
                                const void *V, const double *scores, int k, int32_t *idx,
                                void *out, void *ws, hipStream_t s, void *S_newest = nullptr,
                                const int32_t *cand = nullptr, int n_cand = 0);
// the whole decode step in one kernel (one workgroup per pair); usable when
// step_single_kernel() says so (bf16, enough pairs to cover the chip)
bool step_single_kernel(const Geo &g, int k, int num_cu);
// the whole fp32 decode step in one kernel (a few workgroups per pair) for
// steps of small per-pair bytes (contiguous caches); its workspace
bool step_f32_single_kernel(const Geo &g, int k);
size_t step_f32_ws_bytes(const Geo &g, int k);
hipError_t launch_decode_step_f32(const Geo &g, const void *q, const void *K, const void *V,
                                  void *S, double *scores, int k, int32_t *idx, void *out,
                                  void *ws, hipStream_t s);
// the arrival words of a plan's in-kernel combine (the start of ws;
// nullptr: the plan has none)
uint64_t *step_ctrl(const AttnPlan &p, void *ws);
// where a two-kernel step keeps its fp64 scores in ws when the caller
// passes no scores buffer (or, with tile candidates, their scores, then
// their block numbers: step_cands_in_ws), and the workspace bytes that form
// needs (k > 0: room for the tile candidates of step_tile_cands(g, k, cu))
double *step_scores_in_ws(const Geo &g, const AttnPlan &p, void *ws);
int32_t *step_cands_in_ws(const Geo &g, const AttnPlan &p, const TileCands &tc, void *ws);
size_t step_ws_with_scores(const Geo &g, const AttnPlan &p, int k = 0, int num_cu = 0);
// Quest-style summaries ([pair][nb_cap][2][head_dim]: minimum, maximum) of
// blocks [j0, j1), and the decode step's first kernel with the Quest bound
// (update: the newest block's rows rebuilt first); bf16
hipError_t launch_quest_summary(const Geo &g, const void *K, void *Sq, int j0, int j1,
                                hipStream_t s);
hipError_t launch_quest_score(const Geo &g, const void *q, const void *K, void *Sq,
                              double *scores, int num_cu, uint64_t *ctrl_zero, bool update,
                              hipStream_t s);
// token-level decode step (every token its own block; bf16): scores from K,
// then select + attend; workspace plan_tok(...).ws_bytes
AttnPlan plan_tok(const Geo &g, int k, int num_cu);
hipError_t launch_tok_step(const Geo &g, const void *q, const void *K, const void *V,
                           double *scores, int k, int32_t *idx, void *out, void *ws, int num_cu,
                           hipStream_t s);
// measurement helper: stream `bytes` (a multiple of 16) of buf, XOR-folding
// them into the 16-byte sink
hipError_t launch_read_probe(const void *buf, size_t bytes, void *sink, int num_cu,
                             hipStream_t s);
// (quest: S holds the Quest-style [pair][nb_cap][2][head_dim] summaries and
// the blocks are ranked by the Quest bound; contiguous caches only)
hipError_t launch_decode_step(const Geo &g, const void *q, const void *K, const void *V, void *S,
                              double *scores, int k, int32_t *idx, void *out, int num_cu,
                              hipStream_t s, bool quest = false);

// ---------------------------------------------------------------------------
// device helpers (bf16 is carried as its raw 16 bits)
// ---------------------------------------------------------------------------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// One 16-byte global load of data read once (nontemporal hint: streamed
// through without displacing reusable lines).
__device__ __forceinline__ u32x4 ld_nt16(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs): adding
// 0x7FFF plus the lowest kept bit carries into the kept half exactly when
// the dropped half is above one half, or equal to it with an odd kept half.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

}  // namespace kin
