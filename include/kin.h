/*
 * kin.h -- C ABI of libkin.so: block top-k sparse decode attention for
 * AMD Instinct MI355X (gfx950), hand-written HIP.
 *
 * The method (sources: the skill summary page "Kinetics: Memory-Aware
 * Test-Time Scaling", section "Implementation", module BlockTopKAttention;
 * the rebuttal page "Kinetics: Rethinking Test-Time Scaling Law", answers
 * Q4 "KV block size and grouping strategy", "W2. Alternative sparse
 * attention variants" and "W2 & Q2: Real-world latency benchmarks"):
 * at every decode step each sequence brings one new query per head and
 * attends to its whole retained KV cache.  The cache is cut into KV blocks
 * of `block` tokens; each block is represented by the mean of its keys; the
 * query (all heads of one GQA group together) scores every representative,
 * the k best blocks are kept, and exact softmax(q.k / sqrt(d)) . v runs over
 * the kept blocks' tokens only.  The KV budget in tokens is block * k.
 *
 * Readings of points the pages leave open:
 *   - representative: the mean key (for one query, q.mean(k) equals the
 *     page's "mean score per block");
 *   - one selection per (sequence, KV head), shared by its query heads; the
 *     group's block score is the SUM of the heads' scores, computed in fp64
 *     without the 1/sqrt(d) factor (it does not change the order);
 *   - ties keep the lower block index; indices come out ascending;
 *   - a partial last block is averaged over its valid tokens;
 *   - the new token is already in the cache: attention covers [0, ctx_len).
 *
 * Shapes and layouts (all row-major, contiguous, device memory):
 *   hq = hkv * gqa;  query head h reads KV head h / gqa
 *   nb = ceil(ctx_len / block),  nb_cap = ceil(t_cap / block)
 *   q, out   [batch][hq][head_dim]            dtype
 *   K, V     [batch][hkv][t_cap][head_dim]    dtype
 *   S        [batch][hkv][nb_cap][head_dim]   dtype (block summaries)
 *   scores   [batch][hkv][nb_cap]             double
 *   idx      [batch][hkv][k]                  int32
 * dtype KIN_F32 (binary32) or KIN_BF16 (bfloat16) applies to q, K, V, S
 * and out alike.  Supported: head_dim 128; block 16, 32, 64 or 128;
 * 1 <= gqa <= 16; nb <= 16384.
 *
 * Besides the block method on contiguous caches, the library has decode
 * steps for variable lengths and paged caches (kin_paged_*), for prompts
 * shared by Best-of-N samples (kin_shared_decode_step), for blocks of one
 * token (kin_token_decode_step) and for a Quest-style representative
 * (kin_quest_*), each documented where it is declared below.
 *
 * Conventions for every call:
 *   - The caller owns every buffer; the library allocates nothing, never
 *     synchronises, and keeps no state beyond cached device properties and a
 *     thread-local error message.  Outputs must not alias inputs.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream
 *     of the current device) in call order; calls return before it runs.
 *   - Arguments are checked on the host before anything is enqueued; a bad
 *     argument returns its code, kin_last_error() describes it, and nothing
 *     runs.  A failed launch returns KIN_ERR_HIP.  Faults inside a kernel
 *     surface at the caller's next synchronisation, as with any HIP work.
 *   - Pointers must be 16-byte aligned.  The values read must be finite.
 *   - No C++ exception crosses this interface.
 *   - The calls launch kernels only (no memset, copy or allocation), so they
 *     can be captured into a HIP graph and replayed.
 *   - Workspaces (`ws`): a workspace must be ZERO-FILLED ONCE before its
 *     first use (hipMemset, or a zero-initialised allocation).  Its first
 *     8 KiB hold one 64-bit arrival word per (sequence, KV head) pair, in
 *     which the workgroups that split a pair's kept blocks count themselves
 *     so that the last one combines their partial results; every call
 *     leaves those words at zero when it completes, so a workspace zeroed
 *     once stays valid for every later call and graph replay, of any shape,
 *     through any entry point.  The rest of a workspace needs no clearing.
 *     Calls that overlap in time must not share a workspace.
 */
#ifndef KIN_H
#define KIN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KIN_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define KIN_API __attribute__((visibility("default")))
#else
#define KIN_API
#endif

typedef void *kin_stream; /* a hipStream_t */

typedef enum kin_dtype {
    KIN_F32 = 0,
    KIN_BF16 = 1
} kin_dtype;

typedef enum kin_status {
    KIN_OK = 0,
    KIN_ERR_NULL = -1,        /* a required pointer is NULL */
    KIN_ERR_SHAPE = -2,       /* a size or range is out of bounds */
    KIN_ERR_DTYPE = -3,       /* dtype is not KIN_F32 or KIN_BF16 */
    KIN_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    KIN_ERR_UNSUPPORTED = -5, /* valid, but not built (e.g. head_dim != 128) */
    KIN_ERR_WORKSPACE = -6,   /* workspace too small */
    KIN_ERR_HIP = -7          /* the HIP runtime refused a launch */
} kin_status;

typedef struct kin_desc {
    int32_t batch;    /* sequences in the decode batch */
    int32_t hkv;      /* KV heads */
    int32_t gqa;      /* query heads per KV head */
    int32_t head_dim; /* channels per head (128) */
    int32_t t_cap;    /* cache capacity in tokens per (sequence, KV head) */
    int32_t ctx_len;  /* valid tokens: [0, ctx_len), 1 <= ctx_len <= t_cap */
    int32_t block;    /* KV block size in tokens */
    int32_t dtype;    /* kin_dtype */
} kin_desc;

/* Block summaries (the block representative: mean key).
 * Defining passages: the skill summary page "Kinetics: Memory-Aware
 * Test-Time Scaling", section "Implementation" (BlockTopKAttention divides
 * the sequence into blocks and ranks each block by the mean of its
 * attention scores; for one query that mean equals q . (mean key of the
 * block), so the mean key is the block's representative), and the rebuttal
 * page "Kinetics: Rethinking Test-Time Scaling Law", answer "Q4: KV block
 * size and grouping strategy" (blocks of 16, 32 or 64 KV tokens).
 * Recomputes from scratch every block that intersects [t_begin, t_end) and
 * [0, ctx_len): S[b][g][j][c] = round(sum_{t in block j, t < ctx_len}
 * K[b][g][t][c] / n_j), n_j = min(block, ctx_len - j*block), the sum taken
 * in fp64 in ascending t, rounded fp64 -> fp32 (RNE) and, for bf16, fp32 ->
 * bf16 (RNE).  After prefill call it with [0, ctx_len); at a decode step,
 * after appending token ctx_len-1, with [ctx_len-1, ctx_len).  Other blocks
 * of S are not touched.  Idempotent.
 * Errors: NULL pointers; 0 <= t_begin <= t_end <= t_cap violated. */
KIN_API kin_status kin_block_summary_update(const kin_desc *desc, const void *K, void *S,
                                    int32_t t_begin, int32_t t_end, kin_stream stream);

/* Block scores.  Defining passages: the skill summary page "Kinetics:
 * Memory-Aware Test-Time Scaling", section "Implementation" (the mean score
 * per block of BlockTopKAttention, which ranks the blocks), and the
 * rebuttal page "Kinetics: Rethinking Test-Time Scaling Law", answer "Q4:
 * KV block size and grouping strategy" (Block-TopK groups the KV cache into
 * fixed-size blocks and scores each block as a whole).  The pages do not
 * say how a GQA group's heads combine; the reading taken is the sum of the
 * heads' scores, one selection per KV head.
 * scores[b][g][j] = sum over the group's query heads h
 * (h / gqa == g) of q[b][h] . S[b][g][j], in fp64, for j < nb; -0.0 is
 * written as +0.0.  Entries j >= nb are not written.
 * Errors: NULL pointers, shape. */
KIN_API kin_status kin_block_score(const kin_desc *desc, const void *q, const void *S, double *scores,
                           kin_stream stream);

/* Top-k block selection.  Defining passages: the skill summary page
 * "Kinetics: Memory-Aware Test-Time Scaling", section "Implementation"
 * (BlockTopKAttention keeps the top-k blocks by their block scores), and the
 * rebuttal page "Kinetics: Rethinking Test-Time Scaling Law", answer "Q4: KV
 * block size and grouping strategy" (the KV budget is block size x number of
 * kept blocks, e.g. (16, 64), (32, 32), (64, 16) for 1024 tokens).
 * idx[b][g][0..k) = the min(k, nb) block indices
 * with the largest scores, ties to the lower index, in ascending order,
 * followed by -1 when k > nb.  Only scores[b][g][0..nb) are read.
 * Errors: NULL pointers; k < 1; nb > 16384 (unsupported). */
KIN_API kin_status kin_block_topk(const kin_desc *desc, const double *scores, int32_t k, int32_t *idx,
                          kin_stream stream);

/* Sparse decode attention.  Defining passage: the skill summary page
 * "Kinetics: Memory-Aware Test-Time Scaling", section "Implementation"
 * (BlockTopKAttention masks every token outside the kept blocks, then takes
 * the softmax of q.k / sqrt(d) and multiplies by V; the masked tokens have
 * weight zero, so the result is the softmax over the kept tokens alone).
 * For each query head h of KV head g:
 * out[b][h] = sum_t softmax_t(q[b][h] . K[b][g][t] / sqrt(head_dim)) V[b][g][t]
 * over the tokens t < ctx_len of the blocks listed in idx[b][g][0..k)
 * (entries < 0 or >= nb are skipped).  Accumulation is fp32.
 * `ws` is scratch of at least kin_sparse_ws_bytes(desc, k) bytes (may be
 * NULL when that is 0), zero-filled once before its first use (see the
 * conventions above).
 * Errors: NULL pointers, shape, workspace. */
KIN_API kin_status kin_sparse_decode_attn(const kin_desc *desc, const void *q, const void *K,
                                  const void *V, const int32_t *idx, int32_t k, void *out,
                                  void *ws, size_t ws_bytes, kin_stream stream);

/* Dense decode attention over every token in [0, ctx_len).  Defining
 * passage: the rebuttal page "Kinetics: Rethinking Test-Time Scaling Law",
 * answer "W2 & Q2: Real-world latency benchmarks" (decode latency per step
 * of dense attention against Block-TopK at a 32K-token KV cache): this is
 * that dense comparison, the same softmax(q.k / sqrt(d)) . v over every
 * token.  Same conventions as kin_sparse_decode_attn. */
KIN_API kin_status kin_dense_decode_attn(const kin_desc *desc, const void *q, const void *K,
                                 const void *V, void *out, void *ws, size_t ws_bytes,
                                 kin_stream stream);

/* The two halves of a decode step, each one fused kernel.
 * kin_decode_update_score = kin_block_summary_update over
 * [ctx_len-1, ctx_len) followed by kin_block_score (the newest block's
 * summary is rebuilt and scored in the same launch as every other block).
 * kin_decode_select_attend = kin_block_topk followed by
 * kin_sparse_decode_attn (each pair's workgroup selects its blocks into LDS
 * and attends over them; idx still receives the selection).  Workspace as
 * for kin_sparse_decode_attn (kin_sparse_ws_bytes).  Same errors as the
 * calls they stand for. */
KIN_API kin_status kin_decode_update_score(const kin_desc *desc, const void *q, const void *K,
                                           void *S, double *scores, kin_stream stream);
KIN_API kin_status kin_decode_select_attend(const kin_desc *desc, const void *q, const void *K,
                                            const void *V, const double *scores, int32_t k,
                                            int32_t *idx, void *out, void *ws, size_t ws_bytes,
                                            kin_stream stream);

/* One whole sparse decode step, enqueued on `stream`: summary update of
 * the newest block ([ctx_len-1, ctx_len)), scores, top-k and sparse
 * attention, with the same results as those four calls in sequence.  S is
 * updated in place; scores and idx receive the step's intermediate
 * results.  scores may be NULL: the scores are then not written (the
 * single-kernel form keeps them in LDS; the two-kernel form keeps them in
 * ws, which must then hold kin_sparse_ws_bytes(desc, k) bytes, or, with
 * more than 4096 blocks per pair and one length for every sequence, keeps
 * there only each score tile's own k best blocks, a superset of the
 * pair's top k).  With bf16 data and at least as many (sequence, KV head)
 * pairs as the device has compute units it is ONE kernel (a workgroup per
 * pair runs all four steps, the scores never leave LDS before the
 * selection); otherwise it is two kernels, those of kin_decode_update_score
 * then kin_decode_select_attend (handing over the tiles' candidates instead
 * of every score when it does), plus a combine pass when a pair's kept
 * blocks are split over several workgroups. */
KIN_API kin_status kin_sparse_decode_step(const kin_desc *desc, const void *q, const void *K,
                                  const void *V, void *S, double *scores, int32_t k,
                                  int32_t *idx, void *out, void *ws, size_t ws_bytes,
                                  kin_stream stream);

/* The same step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace argument: the workspace kin_sparse_decode_step
 * would need comes from a scratch array that the library holds on every
 * device it runs on, KIN_NOALLOC_SCRATCH_BYTES bytes, kept until the
 * process ends.  The call itself allocates nothing (no hipMalloc, no
 * allocating library routine).  Results equal kin_sparse_decode_step's on
 * the same arguments.  A step that needs more scratch than the array holds
 * (few (sequence, KV head) pairs with very many blocks and no scores
 * buffer, e.g. 200 pairs of 16384 blocks) returns KIN_ERR_WORKSPACE before
 * anything is enqueued.  Every call on a device shares that device's array:
 * calls that overlap in time on one device (other streams, other host
 * threads) race and must be serialised by the caller.  Errors: as
 * kin_sparse_decode_step. */
#define KIN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
KIN_API kin_status kin_sparse_decode_step_noalloc(const kin_desc *desc, const void *q,
                                                  const void *K, const void *V, void *S,
                                                  double *scores, int32_t k, int32_t *idx,
                                                  void *out, kin_stream stream);

/* ---- Variable lengths and paged caches ---------------------------------
 * The serving layout of the latency runs on the rebuttal page "Kinetics:
 * Rethinking Test-Time Scaling Law" (W2 & Q2: Real-world latency
 * benchmarks: sequences of about 32K tokens that differ by a few thousand,
 * a paged KV cache): every sequence has its own length and K/V live in
 * fixed-size pages of a shared pool.  bf16 only.
 *
 * kin_pages (all device pointers; the struct itself is host memory):
 *   ctx_lens    [batch] int32 tokens of each sequence, or NULL: every
 *               sequence holds desc->ctx_len tokens.  desc->ctx_len is then
 *               an upper bound; entries are clamped to [1, desc->ctx_len].
 *   page_table  [batch][max_pages] int32: page p of sequence b holds its
 *               tokens [p * page_size, (p + 1) * page_size); or NULL: K and
 *               V are the contiguous [batch][hkv][t_cap][head_dim] caches.
 *               Entries outside [0, num_pages) are clamped into the pool.
 *   page_size   tokens per page: a power of two, >= 16, a multiple of block
 *               (so a KV block never straddles two pages).
 *   max_pages   columns of page_table; desc->t_cap = max_pages * page_size.
 *   num_pages   pages in the pools.
 * Paged K and V pools: [num_pages][hkv][page_size][head_dim].  The summaries
 * S stay contiguous, [batch][hkv][nb_cap][head_dim], nb_cap from t_cap.
 *
 * kin_paged_summary_update: as kin_block_summary_update, over the blocks of
 * [t_begin, t_end) inside each sequence's own length.
 * kin_paged_decode_step: as kin_sparse_decode_step, each sequence with its
 * own length (its newest block is the one holding its last token); k <=
 * 2048; workspace kin_sparse_ws_bytes(desc, k).  scores entries past a
 * sequence's own block count are unspecified.  Errors: as the contiguous
 * calls, plus KIN_ERR_UNSUPPORTED for fp32 or k > 2048 and KIN_ERR_SHAPE for
 * a page geometry that breaks the rules above. */
typedef struct kin_pages {
    const int32_t *ctx_lens;
    const int32_t *page_table;
    int32_t page_size;
    int32_t max_pages;
    int32_t num_pages;
} kin_pages;

KIN_API kin_status kin_paged_summary_update(const kin_desc *desc, const kin_pages *pages,
                                            const void *K, void *S, int32_t t_begin,
                                            int32_t t_end, kin_stream stream);
KIN_API kin_status kin_paged_decode_step(const kin_desc *desc, const kin_pages *pages,
                                         const void *q, const void *K, const void *V, void *S,
                                         double *scores, int32_t k, int32_t *idx, void *out,
                                         void *ws, size_t ws_bytes, kin_stream stream);

/* Shared-prompt Best-of-N decode step.  The N samples of a prompt share its
 * first prompt_len tokens (the prompt), whose K/V and block summaries are
 * stored once per prompt, so their rows are read once for all N samples
 * (rebuttal page "Kinetics: Rethinking Test-Time Scaling Law", W2 & Q2:
 * Best-of-N decode batches; the prompt is common to the N samples).
 * Sequences b = p * n_share .. p * n_share + n_share - 1 share prompt p.
 *   Kp, Vp  [batch / n_share][hkv][prompt_len][head_dim], bf16: the prompts'
 *           keys and values (read only);
 *   Sp      [batch / n_share][hkv][prompt_len / block][head_dim]: the prompts'
 *           block summaries (kin_block_summary_update on Kp with batch =
 *           batch / n_share and t_cap = ctx_len = prompt_len builds them);
 *   K, V, S as for kin_sparse_decode_step; their rows for tokens below
 *           prompt_len (blocks below prompt_len / block) are never read.
 * Each sequence's tokens [0, prompt_len) come from its prompt and
 * [prompt_len, ctx_len) from its own cache; everything else is
 * kin_sparse_decode_step (the newest block is always the sequence's own).
 * Workspace kin_sparse_ws_bytes(desc, k).  bf16 only; prompt_len a multiple
 * of desc->block, at least one block and below desc->ctx_len; n_share
 * divides batch; k <= 2048.  Errors: as kin_sparse_decode_step, plus
 * KIN_ERR_SHAPE for a share that breaks these rules and
 * KIN_ERR_UNSUPPORTED for fp32 or k > 2048. */
typedef struct kin_shared_prompt {
    int32_t n_share;
    int32_t prompt_len;
    const void *Kp;
    const void *Vp;
    const void *Sp;
} kin_shared_prompt;

KIN_API kin_status kin_shared_decode_step(const kin_desc *desc, const kin_shared_prompt *share,
                                          const void *q, const void *K, const void *V, void *S,
                                          double *scores, int32_t k, int32_t *idx, void *out,
                                          void *ws, size_t ws_bytes, kin_stream stream);

/* Quest-style representative.  The rebuttal page "Kinetics: Rethinking
 * Test-Time Scaling Law" (Q4 "KV block size and grouping strategy", and W2)
 * names Quest as the second grouping strategy beside Block-TopK without
 * defining it; it is read as the published Quest criterion.  Each block is
 * boxed by the channel-wise minimum and maximum of its keys,
 *   Sq [batch][hkv][nb_cap][2][head_dim], cache dtype: row 0 the minimum,
 *      row 1 the maximum (over the block's tokens below ctx_len; exact, no
 *      rounding),
 * and ranked by the largest q.k inside the box, summed over the GQA group's
 * heads: score_j = sum_h sum_c max(q_hc * min_jc, q_hc * max_jc), fp64.
 * Selection (ties to the lower index) and attention are those of the block
 * method.
 *
 * kin_quest_summary_update: the two rows of every block meeting [t_begin,
 * t_end) and [0, ctx_len).
 * kin_quest_decode_step: rebuilds the newest block's two rows, scores every
 * block with the bound, keeps the k best, attends over them (one kernel on
 * `stream` when batch * hkv covers the device's compute units, else two).
 * scores: NULL or [batch][hkv][nb_cap] fp64 (entries < nb).
 * Workspace: kin_quest_ws_bytes(desc, k) bytes.  bf16 only; k <= 2048.
 * Errors: as kin_sparse_decode_step, plus KIN_ERR_UNSUPPORTED for fp32 or
 * k > 2048. */
KIN_API kin_status kin_quest_summary_update(const kin_desc *desc, const void *K, void *Sq,
                                            int32_t t_begin, int32_t t_end, kin_stream stream);
KIN_API kin_status kin_quest_decode_step(const kin_desc *desc, const void *q, const void *K,
                                         const void *V, void *Sq, double *scores, int32_t k,
                                         int32_t *idx, void *out, void *ws, size_t ws_bytes,
                                         kin_stream stream);
KIN_API size_t kin_quest_ws_bytes(const kin_desc *desc, int32_t k);

/* Token-level top-k decode step: every token is its own block (desc->block
 * must be 1), so the keys are their own representatives and there is no
 * summary array.  TopK attention over single tokens is the variant the
 * rebuttal page "Kinetics: Rethinking Test-Time Scaling Law" (Q2) sets
 * beside Block-TopK; here it is the block method with blocks of one token.
 * Per (sequence, KV head): score_t = sum over the group's query heads of
 * q_h . K[t] in fp64 for t < ctx_len; the k tokens with the largest scores
 * (ties to the lower index) are written to idx[b][hkv][k] ascending, -1 past
 * min(k, ctx_len); out = softmax(q . k / sqrt(d)) . v over the kept tokens.
 *   K, V      [batch][hkv][t_cap][head_dim], bf16 (read only).
 *   scores    NULL, or [batch][hkv][t_cap] fp64: entries t < ctx_len get the
 *             scores (the others are left alone).
 *   ws        kin_token_ws_bytes(desc, k) bytes of device scratch (the
 *             two-kernel form keeps there the scores' top words, its count
 *             tables and, with several workgroups per pair, what they
 *             exchange during the selection; when every score tile of a
 *             pair first keeps its own k best tokens, only those
 *             candidates' top words and token numbers).
 * bf16 only; 1 <= k <= 8192; ctx_len <= 262144.  Errors: KIN_ERR_SHAPE for
 * block != 1 or k < 1, KIN_ERR_UNSUPPORTED for fp32, k > 8192 or longer
 * contexts, plus the checks of the other calls.  One kernel on `stream` when
 * batch * hkv covers the device's compute units, ctx_len <= 32768 and k <=
 * 2048 (no per-token score is written unless scores is given); two kernels
 * otherwise. */
KIN_API kin_status kin_token_decode_step(const kin_desc *desc, const void *q, const void *K,
                                         const void *V, double *scores, int32_t k, int32_t *idx,
                                         void *out, void *ws, size_t ws_bytes, kin_stream stream);
KIN_API size_t kin_token_ws_bytes(const kin_desc *desc, int32_t k);

/* Workspace sizes in bytes (0 when none is needed); -1 cast to size_t on
 * a bad descriptor.  kin_sparse_ws_bytes covers both kin_sparse_decode_attn
 * and kin_sparse_decode_step (also with scores == NULL).  Sizes depend on the current device's
 * compute-unit count: query them on the device the calls will run on. */
KIN_API size_t kin_sparse_ws_bytes(const kin_desc *desc, int32_t k);
KIN_API size_t kin_dense_ws_bytes(const kin_desc *desc);

/* Measurement helper, not a step of the method: stream `bytes` bytes of the
 * device buffer `buf` with plain 16-byte reads (every word once) on `stream`,
 * as a measured read-bandwidth ceiling to quote the decode step against,
 * next to the published peak.  The reads are XOR-folded into the 16-byte
 * device buffer `sink` (four 32-bit words, XOR-accumulated: zero it first to
 * read the buffer's XOR back).  buf and sink 16-byte aligned; bytes a
 * positive multiple of 16 (KIN_ERR_SHAPE otherwise). */
KIN_API kin_status kin_hbm_read_probe(const void *buf, size_t bytes, void *sink,
                                      kin_stream stream);

/* Name of a status code, and the detail of the last error on this thread. */
KIN_API const char *kin_status_str(kin_status status);
KIN_API const char *kin_last_error(void);
KIN_API int32_t kin_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KIN_H */
