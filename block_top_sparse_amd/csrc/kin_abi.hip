// kin_abi.hip -- the C ABI of libkin.so (declared in include/kin.h):
// argument checks on the host, workspace sizing, launches on the caller's
// stream.  Nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdlib.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kin_internal.h"

namespace {

thread_local char g_last_error[512] = "";

kin_status fail(kin_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

kin_status ok() {
    g_last_error[0] = '\0';
    return KIN_OK;
}

// compute-unit count per device, read once
constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cu[kMaxDevices];

int num_cu() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_num_cu[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    g_num_cu[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Validate a descriptor and derive the geometry.
kin_status check_desc(const kin_desc *d, kin::Geo *g) {
    if (!d) return fail(KIN_ERR_NULL, "desc is NULL");
    if (d->dtype != KIN_F32 && d->dtype != KIN_BF16)
        return fail(KIN_ERR_DTYPE, "dtype %d is not KIN_F32 (0) or KIN_BF16 (1)", d->dtype);
    if (d->batch < 1 || d->hkv < 1 || d->gqa < 1)
        return fail(KIN_ERR_SHAPE, "batch %d, hkv %d and gqa %d must be >= 1", d->batch, d->hkv,
                    d->gqa);
    if (d->block < 1)
        return fail(KIN_ERR_SHAPE, "block %d must be >= 1", d->block);
    if (d->t_cap < 1 || d->ctx_len < 1 || d->ctx_len > d->t_cap)
        return fail(KIN_ERR_SHAPE, "need 1 <= ctx_len (%d) <= t_cap (%d)", d->ctx_len, d->t_cap);
    if (d->head_dim != kin::kHeadDim)
        return fail(KIN_ERR_UNSUPPORTED, "head_dim %d: only %d is built", d->head_dim,
                    kin::kHeadDim);
    if (d->block != 16 && d->block != 32 && d->block != 64 && d->block != 128)
        return fail(KIN_ERR_UNSUPPORTED, "block %d: only 16, 32, 64 and 128 are built", d->block);
    if (d->gqa > kin::kMaxGqa)
        return fail(KIN_ERR_UNSUPPORTED, "gqa %d: at most %d query heads per KV head", d->gqa,
                    kin::kMaxGqa);
    const long long pairs = (long long)d->batch * d->hkv;
    if (pairs > 65535 || (long long)d->batch * d->hkv * d->gqa > (1LL << 30))
        return fail(KIN_ERR_UNSUPPORTED, "batch x hkv = %lld pairs: at most 65535", pairs);
    g->batch = d->batch;
    g->hkv = d->hkv;
    g->gqa = d->gqa;
    g->hq = d->hkv * d->gqa;
    g->t_cap = d->t_cap;
    g->ctx_len = d->ctx_len;
    g->block = d->block;
    g->dtype = d->dtype;
    g->nb = (d->ctx_len + d->block - 1) / d->block;
    g->nb_cap = (d->t_cap + d->block - 1) / d->block;
    g->pairs = (int)pairs;
    return KIN_OK;
}

#define KIN_REQUIRE_PTR(p)                                                     \
    do {                                                                       \
        if (!(p)) return fail(KIN_ERR_NULL, "%s is NULL", #p);                 \
        if (!aligned16(p)) return fail(KIN_ERR_ALIGN, "%s is not 16-byte aligned", #p); \
    } while (0)

kin_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(KIN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

// Shared checks of the decode-step entry points.
static kin_status check_step(const kin_desc *desc, kin::Geo *g) {
    kin_status st = check_desc(desc, g);
    if (st != KIN_OK) return st;
    if (g->nb > kin::kMaxBlocks)
        return fail(KIN_ERR_UNSUPPORTED, "%d blocks: at most %d", g->nb, kin::kMaxBlocks);
    return KIN_OK;
}

static kin_status check_ws_size(size_t need, const void *ws, size_t ws_bytes) {
    if (need == 0) return KIN_OK;
    if (!ws) return fail(KIN_ERR_NULL, "ws is NULL but %zu bytes are needed", need);
    if (!aligned16(ws)) return fail(KIN_ERR_ALIGN, "ws is not 16-byte aligned");
    if (ws_bytes < need)
        return fail(KIN_ERR_WORKSPACE, "ws has %zu bytes, %zu needed", ws_bytes, need);
    return KIN_OK;
}

static kin_status check_ws(const kin::AttnPlan &p, const void *ws, size_t ws_bytes) {
    return check_ws_size(p.ws_bytes, ws, ws_bytes);
}

// ---- the step without allocation --------------------------------------
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc) take
// kin_sparse_decode_step's workspace from this file-scope device array:
// KIN_NOALLOC_SCRATCH_BYTES on every device the library runs on, held until
// the process ends.  In host code `scratch` only names the symbol; its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[KIN_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device

// zero n 64-bit words (the arrival words of a fresh scratch array)
__global__ void k_zero_words(uint64_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0ull;
}

// This device's scratch address; on the first call for a device it is
// looked up and the arrival words at its start are cleared on `stream`
// (the array starts zeroed anyway; every call leaves those words at zero).
kin_status scratch_on_device(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KIN_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(KIN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KIN_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        constexpr int n = kin::kCtrlWords;
        k_zero_words<<<(n + 255) / 256, 256, 0, stream>>>(static_cast<uint64_t *>(p), n);
        e = hipGetLastError();
        if (e != hipSuccess)
            return fail(KIN_ERR_HIP, "clearing the scratch words: %s", hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return KIN_OK;
}

}  // namespace

extern "C" {

kin_status kin_block_summary_update(const kin_desc *desc, const void *K, void *S,
                                    int32_t t_begin, int32_t t_end, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_desc(desc, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(S);
    if (t_begin < 0 || t_end < t_begin || t_end > g.t_cap)
        return fail(KIN_ERR_SHAPE, "need 0 <= t_begin (%d) <= t_end (%d) <= t_cap (%d)", t_begin,
                    t_end, g.t_cap);
    const int te = t_end < g.ctx_len ? t_end : g.ctx_len;
    if (t_begin >= te) return ok();  // nothing inside [0, ctx_len)
    const int j0 = t_begin / g.block, j1 = (te - 1) / g.block + 1;
    return launched(kin::launch_block_summary(g, K, S, j0, j1, (hipStream_t)stream),
                    "kin_block_summary_update");
}

kin_status kin_block_score(const kin_desc *desc, const void *q, const void *S, double *scores,
                           kin_stream stream) {
    kin::Geo g;
    kin_status st = check_desc(desc, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(S);
    KIN_REQUIRE_PTR(scores);
    if (g.nb > kin::kMaxBlocks)
        return fail(KIN_ERR_UNSUPPORTED, "%d blocks: at most %d", g.nb, kin::kMaxBlocks);
    return launched(kin::launch_block_score(g, q, S, scores, num_cu(), (hipStream_t)stream),
                    "kin_block_score");
}

kin_status kin_block_topk(const kin_desc *desc, const double *scores, int32_t k, int32_t *idx,
                          kin_stream stream) {
    kin::Geo g;
    kin_status st = check_desc(desc, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(scores);
    KIN_REQUIRE_PTR(idx);
    if (k < 1) return fail(KIN_ERR_SHAPE, "k = %d: need k >= 1", k);
    if (g.nb > kin::kMaxBlocks)
        return fail(KIN_ERR_UNSUPPORTED, "%d blocks: at most %d", g.nb, kin::kMaxBlocks);
    return launched(kin::launch_block_topk(g, scores, k, idx, (hipStream_t)stream),
                    "kin_block_topk");
}

static kin_status attention(const kin_desc *desc, const void *q, const void *K, const void *V,
                            const int32_t *idx, int32_t k, void *out, void *ws,
                            size_t ws_bytes, kin_stream stream, bool dense) {
    kin::Geo g;
    kin_status st = check_desc(desc, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(V);
    KIN_REQUIRE_PTR(out);
    if (!dense) {
        KIN_REQUIRE_PTR(idx);
        if (k < 1) return fail(KIN_ERR_SHAPE, "k = %d: need k >= 1", k);
    }
    const kin::AttnPlan p = kin::plan_attention(g, dense ? 0 : k, dense, num_cu());
    st = check_ws(p, ws, ws_bytes);
    if (st != KIN_OK) return st;
    return launched(kin::launch_attention(g, p, q, K, V, dense ? nullptr : idx, k, out, ws,
                                          (hipStream_t)stream),
                    dense ? "kin_dense_decode_attn" : "kin_sparse_decode_attn");
}

kin_status kin_sparse_decode_attn(const kin_desc *desc, const void *q, const void *K,
                                  const void *V, const int32_t *idx, int32_t k, void *out,
                                  void *ws, size_t ws_bytes, kin_stream stream) {
    return attention(desc, q, K, V, idx, k, out, ws, ws_bytes, stream, false);
}

kin_status kin_dense_decode_attn(const kin_desc *desc, const void *q, const void *K,
                                 const void *V, void *out, void *ws, size_t ws_bytes,
                                 kin_stream stream) {
    return attention(desc, q, K, V, nullptr, 0, out, ws, ws_bytes, stream, true);
}

kin_status kin_decode_update_score(const kin_desc *desc, const void *q, const void *K, void *S,
                                   double *scores, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_step(desc, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(S);
    KIN_REQUIRE_PTR(scores);
    return launched(kin::launch_update_and_score(g, q, K, S, scores, num_cu(), (hipStream_t)stream),
                    "kin_decode_update_score");
}

kin_status kin_decode_select_attend(const kin_desc *desc, const void *q, const void *K,
                                    const void *V, const double *scores, int32_t k, int32_t *idx,
                                    void *out, void *ws, size_t ws_bytes, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_step(desc, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(V);
    KIN_REQUIRE_PTR(scores);
    KIN_REQUIRE_PTR(idx);
    KIN_REQUIRE_PTR(out);
    if (k < 1) return fail(KIN_ERR_SHAPE, "k = %d: need k >= 1", k);
    const kin::AttnPlan p = kin::plan_step(g, k, num_cu());
    st = check_ws(p, ws, ws_bytes);
    if (st != KIN_OK) return st;
    return launched(kin::launch_select_attend(g, p, q, K, V, scores, k, idx, out, ws,
                                              (hipStream_t)stream),
                    "kin_decode_select_attend");
}

// Workspace bytes the decode step takes for this geometry (scores: whether
// the caller passes a scores buffer; without one the two-kernel form keeps
// the scores in the workspace).
static size_t step_ws_need(const kin::Geo &g, int32_t k, int cu, bool scores) {
    if (kin::step_single_kernel(g, k, cu)) return 0;
    if (!g.pages && !g.share_n && kin::step_f32_single_kernel(g, k))
        return kin::step_f32_ws_bytes(g, k);
    const kin::AttnPlan p = kin::plan_step(g, k, cu);
    return scores ? p.ws_bytes : kin::step_ws_with_scores(g, p, k, cu);
}

// The decode step for a checked geometry (contiguous or paged).
static kin_status decode_step(const kin::Geo &g, const void *q, const void *K, const void *V,
                              void *S, double *scores, int32_t k, int32_t *idx, void *out,
                              void *ws, size_t ws_bytes, kin_stream stream) {
    kin_status st;
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(V);
    KIN_REQUIRE_PTR(S);
    if (scores && !aligned16(scores))  // NULL: the scores are not returned
        return fail(KIN_ERR_ALIGN, "scores is not 16-byte aligned");
    KIN_REQUIRE_PTR(idx);
    KIN_REQUIRE_PTR(out);
    if (k < 1) return fail(KIN_ERR_SHAPE, "k = %d: need k >= 1", k);
    hipStream_t s = (hipStream_t)stream;
    const int cu = num_cu();
    if (kin::step_single_kernel(g, k, cu))
        return launched(kin::launch_decode_step(g, q, K, V, S, scores, k, idx, out, cu, s),
                        "kin_sparse_decode_step");
    if (!g.pages && !g.share_n && kin::step_f32_single_kernel(g, k)) {
        st = check_ws_size(kin::step_f32_ws_bytes(g, k), ws, ws_bytes);
        if (st != KIN_OK) return st;
        return launched(kin::launch_decode_step_f32(g, q, K, V, S, scores, k, idx, out, ws, s),
                        "kin_sparse_decode_step");
    }
    const kin::AttnPlan p = kin::plan_step(g, k, cu);
    // two kernels hand the scores over in memory: the caller's buffer, or
    // the workspace after the attention's part
    st = check_ws_size(step_ws_need(g, k, cu, scores != nullptr), ws, ws_bytes);
    if (st != KIN_OK) return st;
    double *sc = scores ? scores : kin::step_scores_in_ws(g, p, ws);
    // every block kept and no scores wanted: only the newest summary row is
    // rebuilt, by the fused second half itself (its split partials then count
    // their arrivals in words the previous call on this workspace left at
    // zero)
    const bool newest_only = !scores && k >= g.nb && g.dtype == KIN_BF16;
    if (newest_only && p.fused)
        return launched(kin::launch_select_attend(g, p, q, K, V, sc, k, idx, out, ws, s, S),
                        "kin_sparse_decode_step");
    // no scores wanted, few pairs: the score tiles may hand over only their
    // own k best (kin::step_tile_cands)
    const kin::TileCands tc = scores || newest_only || !p.fused ? kin::TileCands{0, 0, 0}
                                                                : kin::step_tile_cands(g, k, cu);
    int32_t *cand = tc.tiles ? kin::step_cands_in_ws(g, p, tc, ws) : nullptr;
    // the scoring kernel also clears the second kernel's arrival words
    hipError_t e = kin::launch_update_and_score(g, q, K, S, sc, cu, s, newest_only,
                                                kin::step_ctrl(p, ws), cand ? &tc : nullptr,
                                                cand, k);
    if (e == hipSuccess)
        e = kin::launch_select_attend(g, p, q, K, V, sc, k, idx, out, ws, s, nullptr, cand,
                                      tc.n);
    return launched(e, "kin_sparse_decode_step");
}

kin_status kin_sparse_decode_step(const kin_desc *desc, const void *q, const void *K,
                                  const void *V, void *S, double *scores, int32_t k,
                                  int32_t *idx, void *out, void *ws, size_t ws_bytes,
                                  kin_stream stream) {
    // check everything before enqueueing anything
    kin::Geo g;
    kin_status st = check_step(desc, &g);
    if (st != KIN_OK) return st;
    return decode_step(g, q, K, V, S, scores, k, idx, out, ws, ws_bytes, stream);
}

kin_status kin_sparse_decode_step_noalloc(const kin_desc *desc, const void *q, const void *K,
                                          const void *V, void *S, double *scores, int32_t k,
                                          int32_t *idx, void *out, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_step(desc, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(V);
    KIN_REQUIRE_PTR(S);
    if (scores && !aligned16(scores)) return fail(KIN_ERR_ALIGN, "scores is not 16-byte aligned");
    KIN_REQUIRE_PTR(idx);
    KIN_REQUIRE_PTR(out);
    if (k < 1) return fail(KIN_ERR_SHAPE, "k = %d: need k >= 1", k);
    const size_t need = step_ws_need(g, k, num_cu(), scores != nullptr);
    if (need > KIN_NOALLOC_SCRATCH_BYTES)
        return fail(KIN_ERR_WORKSPACE,
                    "this step needs %zu bytes of scratch; the no-allocation step holds %zu "
                    "(use kin_sparse_decode_step with a workspace)",
                    need, (size_t)KIN_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need) {
        st = scratch_on_device((hipStream_t)stream, &ws);
        if (st != KIN_OK) return st;
    }
    return decode_step(g, q, K, V, S, scores, k, idx, out, ws, need ? KIN_NOALLOC_SCRATCH_BYTES : 0,
                       stream);
}

// Variable lengths and paged caches: the descriptor plus the kin_pages
// fields, checked; the kernels read ctx_lens and the page table on the
// device.
static kin_status check_pages(const kin_desc *desc, const kin_pages *pg, kin::Geo *g) {
    kin_status st = check_step(desc, g);
    if (st != KIN_OK) return st;
    if (!pg) return fail(KIN_ERR_NULL, "pages is NULL");
    if (g->dtype != KIN_BF16)
        return fail(KIN_ERR_UNSUPPORTED, "variable lengths and paged caches: bf16 only");
    if (pg->ctx_lens && ((uintptr_t)pg->ctx_lens & 3u))
        return fail(KIN_ERR_ALIGN, "ctx_lens is not 4-byte aligned");
    if (pg->page_table) {
        if ((uintptr_t)pg->page_table & 3u)
            return fail(KIN_ERR_ALIGN, "page_table is not 4-byte aligned");
        const int P = pg->page_size;
        if (P < 16 || (P & (P - 1)) || P < g->block || P % g->block)
            return fail(KIN_ERR_SHAPE,
                        "page_size = %d: need a power of two >= 16, a multiple of block %d", P,
                        g->block);
        if (pg->max_pages < 1 || pg->num_pages < 1)
            return fail(KIN_ERR_SHAPE, "max_pages = %d, num_pages = %d: need >= 1",
                        pg->max_pages, pg->num_pages);
        if ((long long)pg->max_pages * P != g->t_cap)
            return fail(KIN_ERR_SHAPE, "t_cap = %d: need max_pages * page_size = %lld", g->t_cap,
                        (long long)pg->max_pages * P);
        g->pages = pg->page_table;
        g->page_shift = __builtin_ctz((unsigned)P);
        g->max_pages = pg->max_pages;
        g->num_pages = pg->num_pages;
    }
    g->ctx_lens = pg->ctx_lens;
    return KIN_OK;
}

kin_status kin_paged_summary_update(const kin_desc *desc, const kin_pages *pages, const void *K,
                                    void *S, int32_t t_begin, int32_t t_end, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_pages(desc, pages, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(S);
    if (t_begin < 0 || t_end < t_begin || t_end > g.t_cap)
        return fail(KIN_ERR_SHAPE, "need 0 <= t_begin (%d) <= t_end (%d) <= t_cap (%d)", t_begin,
                    t_end, g.t_cap);
    return launched(kin::launch_block_summary_paged(g, K, S, t_begin, t_end, (hipStream_t)stream),
                    "kin_paged_summary_update");
}

kin_status kin_paged_decode_step(const kin_desc *desc, const kin_pages *pages, const void *q,
                                 const void *K, const void *V, void *S, double *scores,
                                 int32_t k, int32_t *idx, void *out, void *ws, size_t ws_bytes,
                                 kin_stream stream) {
    kin::Geo g;
    kin_status st = check_pages(desc, pages, &g);
    if (st != KIN_OK) return st;
    if (k > kin::kStepIdxCap)
        return fail(KIN_ERR_UNSUPPORTED, "k = %d: paged steps keep at most %d blocks", k,
                    kin::kStepIdxCap);
    return decode_step(g, q, K, V, S, scores, k, idx, out, ws, ws_bytes, stream);
}

kin_status kin_shared_decode_step(const kin_desc *desc, const kin_shared_prompt *share,
                                  const void *q, const void *K, const void *V, void *S,
                                  double *scores, int32_t k, int32_t *idx, void *out, void *ws,
                                  size_t ws_bytes, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_step(desc, &g);
    if (st != KIN_OK) return st;
    if (!share) return fail(KIN_ERR_NULL, "share is NULL");
    if (g.dtype != KIN_BF16) return fail(KIN_ERR_UNSUPPORTED, "shared prompts: bf16 only");
    if (share->n_share < 1 || g.batch % share->n_share)
        return fail(KIN_ERR_SHAPE, "n_share = %d must divide batch %d", share->n_share, g.batch);
    if (share->prompt_len < g.block || share->prompt_len % g.block ||
        share->prompt_len >= g.ctx_len)
        return fail(KIN_ERR_SHAPE,
                    "prompt_len = %d: need a multiple of block %d, at least one block, below "
                    "ctx_len %d",
                    share->prompt_len, g.block, g.ctx_len);
    if (k > kin::kStepIdxCap)
        return fail(KIN_ERR_UNSUPPORTED, "k = %d: shared-prompt steps keep at most %d blocks", k,
                    kin::kStepIdxCap);
    const void *Kp = share->Kp, *Vp = share->Vp, *Sp = share->Sp;
    KIN_REQUIRE_PTR(Kp);
    KIN_REQUIRE_PTR(Vp);
    KIN_REQUIRE_PTR(Sp);
    g.share_n = share->n_share;
    g.prompt_len = share->prompt_len;
    g.Kp = Kp;
    g.Vp = Vp;
    g.Sp = Sp;
    return decode_step(g, q, K, V, S, scores, k, idx, out, ws, ws_bytes, stream);
}

kin_status kin_quest_summary_update(const kin_desc *desc, const void *K, void *Sq,
                                   int32_t t_begin, int32_t t_end, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_desc(desc, &g);
    if (st != KIN_OK) return st;
    if (g.dtype != KIN_BF16) return fail(KIN_ERR_UNSUPPORTED, "Quest summaries: bf16 only");
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(Sq);
    if (t_begin < 0 || t_end < t_begin || t_end > g.t_cap)
        return fail(KIN_ERR_SHAPE, "need 0 <= t_begin (%d) <= t_end (%d) <= t_cap (%d)", t_begin,
                    t_end, g.t_cap);
    const int te = t_end < g.ctx_len ? t_end : g.ctx_len;
    if (t_begin >= te) return ok();
    return launched(kin::launch_quest_summary(g, K, Sq, t_begin / g.block,
                                              (te - 1) / g.block + 1, (hipStream_t)stream),
                    "kin_quest_summary_update");
}

kin_status kin_quest_decode_step(const kin_desc *desc, const void *q, const void *K,
                                 const void *V, void *Sq, double *scores, int32_t k, int32_t *idx,
                                 void *out, void *ws, size_t ws_bytes, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_step(desc, &g);
    if (st != KIN_OK) return st;
    if (g.dtype != KIN_BF16) return fail(KIN_ERR_UNSUPPORTED, "Quest step: bf16 only");
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(V);
    KIN_REQUIRE_PTR(Sq);
    if (scores && !aligned16(scores)) return fail(KIN_ERR_ALIGN, "scores is not 16-byte aligned");
    KIN_REQUIRE_PTR(idx);
    KIN_REQUIRE_PTR(out);
    if (k < 1) return fail(KIN_ERR_SHAPE, "k = %d: need k >= 1", k);
    if (k > kin::kStepIdxCap)
        return fail(KIN_ERR_UNSUPPORTED, "k = %d: the Quest step keeps at most %d blocks", k,
                    kin::kStepIdxCap);
    const int cu = num_cu();
    hipStream_t s = (hipStream_t)stream;
    if (kin::step_single_kernel(g, k, cu))
        return launched(kin::launch_decode_step(g, q, K, V, Sq, scores, k, idx, out, cu, s, true),
                        "kin_quest_decode_step");
    const kin::AttnPlan p = kin::plan_step(g, k, cu);
    st = check_ws_size(scores ? p.ws_bytes : kin::step_ws_with_scores(g, p), ws, ws_bytes);
    if (st != KIN_OK) return st;
    double *sc = scores ? scores : kin::step_scores_in_ws(g, p, ws);
    hipError_t e = kin::launch_quest_score(g, q, K, Sq, sc, cu, kin::step_ctrl(p, ws), true, s);
    if (e == hipSuccess) e = kin::launch_select_attend(g, p, q, K, V, sc, k, idx, out, ws, s);
    return launched(e, "kin_quest_decode_step");
}

size_t kin_quest_ws_bytes(const kin_desc *desc, int32_t k) {
    kin::Geo g;
    if (check_step(desc, &g) != KIN_OK) return (size_t)-1;
    if (k < 1 || k > kin::kStepIdxCap) {
        fail(KIN_ERR_SHAPE, "k = %d: need 1 <= k <= %d", k, kin::kStepIdxCap);
        return (size_t)-1;
    }
    return kin::step_ws_with_scores(g, kin::plan_step(g, k, num_cu()));
}

// Token-level step: the descriptor with block 1 (every token its own block).
static kin_status check_tok(const kin_desc *desc, int32_t k, kin::Geo *g) {
    if (!desc) return fail(KIN_ERR_NULL, "desc is NULL");
    if (desc->block != 1)
        return fail(KIN_ERR_SHAPE, "block %d: the token-level step takes block = 1", desc->block);
    kin_desc d = *desc;
    d.block = 16;  // the other fields are checked as for the block calls
    kin_status st = check_desc(&d, g);
    if (st != KIN_OK) return st;
    if (g->dtype != KIN_BF16) return fail(KIN_ERR_UNSUPPORTED, "token-level step: bf16 only");
    if (g->ctx_len > kin::kTokMaxLen)
        return fail(KIN_ERR_UNSUPPORTED, "ctx_len %d: the token-level step takes at most %d",
                    g->ctx_len, kin::kTokMaxLen);
    if (k < 1 || k > kin::kTokIdxCap)
        return fail(k < 1 ? KIN_ERR_SHAPE : KIN_ERR_UNSUPPORTED,
                    "k = %d: the token-level step keeps 1 .. %d tokens", k, kin::kTokIdxCap);
    g->block = 1;
    g->nb = g->ctx_len;
    g->nb_cap = g->t_cap;
    return KIN_OK;
}

kin_status kin_token_decode_step(const kin_desc *desc, const void *q, const void *K,
                                 const void *V, double *scores, int32_t k, int32_t *idx,
                                 void *out, void *ws, size_t ws_bytes, kin_stream stream) {
    kin::Geo g;
    kin_status st = check_tok(desc, k, &g);
    if (st != KIN_OK) return st;
    KIN_REQUIRE_PTR(q);
    KIN_REQUIRE_PTR(K);
    KIN_REQUIRE_PTR(V);
    if (scores && !aligned16(scores)) return fail(KIN_ERR_ALIGN, "scores is not 16-byte aligned");
    KIN_REQUIRE_PTR(idx);
    KIN_REQUIRE_PTR(out);
    const int cu = num_cu();
    st = check_ws_size(kin::plan_tok(g, k, cu).ws_bytes, ws, ws_bytes);
    if (st != KIN_OK) return st;
    return launched(kin::launch_tok_step(g, q, K, V, scores, k, idx, out, ws, cu,
                                         (hipStream_t)stream),
                    "kin_token_decode_step");
}

size_t kin_token_ws_bytes(const kin_desc *desc, int32_t k) {
    kin::Geo g;
    if (check_tok(desc, k, &g) != KIN_OK) return (size_t)-1;
    return kin::plan_tok(g, k, num_cu()).ws_bytes;
}

size_t kin_sparse_ws_bytes(const kin_desc *desc, int32_t k) {
    kin::Geo g;
    if (check_desc(desc, &g) != KIN_OK) return (size_t)-1;
    if (k < 1) {
        fail(KIN_ERR_SHAPE, "k = %d: need k >= 1", k);
        return (size_t)-1;
    }
    const int cu = num_cu();
    const size_t a = kin::plan_attention(g, k, false, cu).ws_bytes;
    // the step's two-kernel form, with room for the scores (scores == NULL)
    const size_t b = kin::step_single_kernel(g, k, cu)      ? 0
                     : kin::step_f32_single_kernel(g, k) ? kin::step_f32_ws_bytes(g, k)
                                                         : kin::step_ws_with_scores(g, kin::plan_step(g, k, cu), k, cu);
    return a > b ? a : b;
}

kin_status kin_hbm_read_probe(const void *buf, size_t bytes, void *sink, kin_stream stream) {
    KIN_REQUIRE_PTR(buf);
    KIN_REQUIRE_PTR(sink);
    if (bytes == 0 || bytes % 16)
        return fail(KIN_ERR_SHAPE, "bytes = %zu: need a positive multiple of 16", bytes);
    return launched(kin::launch_read_probe(buf, bytes, sink, num_cu(), (hipStream_t)stream),
                    "kin_hbm_read_probe");
}

size_t kin_dense_ws_bytes(const kin_desc *desc) {
    kin::Geo g;
    if (check_desc(desc, &g) != KIN_OK) return (size_t)-1;
    return kin::plan_attention(g, 0, true, num_cu()).ws_bytes;
}

const char *kin_status_str(kin_status status) {
    switch (status) {
    case KIN_OK: return "KIN_OK";
    case KIN_ERR_NULL: return "KIN_ERR_NULL";
    case KIN_ERR_SHAPE: return "KIN_ERR_SHAPE";
    case KIN_ERR_DTYPE: return "KIN_ERR_DTYPE";
    case KIN_ERR_ALIGN: return "KIN_ERR_ALIGN";
    case KIN_ERR_UNSUPPORTED: return "KIN_ERR_UNSUPPORTED";
    case KIN_ERR_WORKSPACE: return "KIN_ERR_WORKSPACE";
    case KIN_ERR_HIP: return "KIN_ERR_HIP";
    }
    return "KIN_ERR_UNKNOWN";
}

const char *kin_last_error(void) { return g_last_error; }

int32_t kin_version(void) { return KIN_VERSION; }

}  // extern "C"
